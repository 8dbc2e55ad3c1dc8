// Host-side check of two plan decisions of the library: the BCSR schedule
// (bcsr_schedule) and the dispatch order of tile-vector-wise row tiles
// (tvw_row_order).  Input on stdin, one query per line:
//   schedule <mb> <n> <nnzb>   -> "<tn> <row_groups> <kh>"
//   tvw <mtiles> <count_0> ... -> the row tiles in dispatch order
#include <cstdio>
#include <cstring>
#include <vector>

#include "../sparse_dense_matrix_amd/csrc/internal.h"

int main() {
  char what[16];
  while (std::scanf("%15s", what) == 1) {
    if (!std::strcmp(what, "schedule")) {
      int mb;
      long long n, nnzb;
      if (std::scanf("%d %lld %lld", &mb, &n, &nnzb) != 3 || mb < 0) return 2;
      std::vector<int32_t> rp(static_cast<size_t>(mb) + 1, 0);
      rp[mb] = static_cast<int32_t>(nnzb);
      const sdm::BcsrSchedule sc = sdm::bcsr_schedule(rp.data(), mb, n);
      std::printf("%d %d %d\n", sc.tn, sc.row_groups, sc.kh);
    } else if (!std::strcmp(what, "tvw")) {
      long long mtiles;
      if (std::scanf("%lld", &mtiles) != 1 || mtiles < 0) return 2;
      std::vector<int32_t> ptr(static_cast<size_t>(mtiles) + 1, 0);
      for (long long t = 0; t < mtiles; ++t) {
        int c;
        if (std::scanf("%d", &c) != 1) return 2;
        ptr[t + 1] = ptr[t] + c;
      }
      const sdm::vec<int32_t> order = sdm::tvw_row_order(ptr.data(), mtiles);
      for (size_t i = 0; i < order.size(); ++i) std::printf(i ? " %d" : "%d", order[i]);
      std::printf("\n");
    } else {
      return 2;
    }
  }
  return 0;
}
