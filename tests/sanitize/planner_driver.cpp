// Host planner under the sanitizers: builds the plan of every layout file
// given on the command line with several threads, then walks every entry
// point of the planner (step maps, fetch sets, chunk order, dense calls, the
// vision-group order).  A layout file is int64 n, int32 window, int32 ranks,
// int32 order, then the four int32[n] tracks (sample, seg, noise, pos).
// Exit status 0 when every call returns; the sanitizers abort on a finding.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "planner.hpp"

namespace bsm {
void set_error(const std::string& msg) { std::fprintf(stderr, "planner error: %s\n", msg.c_str()); }
}  // namespace bsm

static bool read_all(FILE* f, void* p, size_t bytes) { return std::fread(p, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
  int checked = 0;
  for (int i = 1; i < argc; ++i) {
    FILE* f = std::fopen(argv[i], "rb");
    if (!f) return 2;
    int64_t n = 0;
    int32_t hdr[3];
    if (!read_all(f, &n, sizeof n) || !read_all(f, hdr, sizeof hdr)) return 2;
    std::vector<int32_t> t[4];
    for (auto& v : t) {
      v.resize((size_t)n);
      if (!read_all(f, v.data(), (size_t)n * sizeof(int32_t))) return 2;
    }
    std::fclose(f);
    bsm_plan_desc d{};
    d.n = n;
    d.sample = t[0].data();
    d.seg = t[1].data();
    d.noise = t[2].data();
    d.pos = t[3].data();
    d.window = hdr[0];
    d.ranks = hdr[1];
    d.block = 128;
    d.order = hdr[2];
    d.threads = 8;
    bsm::Plan p;
    if (bsm::build_plan(d, p) != BSM_OK) return 3;
    std::vector<uint8_t> map((size_t)p.tps * p.tps), need((size_t)p.ranks * p.tps);
    int64_t pairs = 0;
    for (int32_t r = 0; r < p.ranks; ++r) {
      for (int32_t s = 0; s < p.ranks; ++s) {
        pairs += bsm::step_map(p, r, s, map.data());
        std::vector<bsm::Call> calls;
        const int rc = bsm::dense_calls(p, r, s, calls);
        if (rc != BSM_OK && !(rc == BSM_E_UNSUPPORTED && !p.pos_rising)) return 4;
      }
      bsm::fetch_set(p, r, need.data());
    }
    if (pairs != p.total_pairs) return 5;
    if (p.order != BSM_ORDER_CONTIGUOUS && p.ranks > 1) {
      std::vector<int32_t> bp((size_t)p.ntiles);
      bsm::ChunkResult cr;
      if (bsm::chunk_order(p, 1, 8, 0.0, 2, bp.data(), cr) != BSM_OK) return 6;
    }
    std::vector<int32_t> perm((size_t)n);
    if (bsm::vision_group_order(n, d.sample, d.seg, perm.data()) != BSM_OK) return 7;
    ++checked;
  }
  std::printf("checked %d layouts\n", checked);
  return 0;
}
