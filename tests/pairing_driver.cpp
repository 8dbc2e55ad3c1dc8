// Host-side check of the BCSR plan's block-row pairing (bcsr_pairing in the
// library): reads a block pattern on stdin, prints the pairs and their units.
// Input:  mb kb nnzb, then row_ptr[mb + 1], then col_idx[nnzb].
// Output: the saving, the pair count, one line per pair (first row, second
//         row, first unit, end unit), the unit count, one line per unit
//         (block column, block of the first row, block of the second).
#include <cstdio>
#include <vector>

#include "../sparse_dense_matrix_amd/csrc/internal.h"

int main() {
  int mb, kb, nnzb;
  if (std::scanf("%d %d %d", &mb, &kb, &nnzb) != 3 || mb < 0 || kb < 0 || nnzb < 0) return 2;
  std::vector<int32_t> rp(static_cast<size_t>(mb) + 1), ci(static_cast<size_t>(nnzb));
  for (auto &x : rp)
    if (std::scanf("%d", &x) != 1) return 2;
  for (auto &x : ci)
    if (std::scanf("%d", &x) != 1) return 2;
  sdm::vec<int32_t> pair_rows, pair_ptr, units;
  const double saving = sdm::bcsr_pairing(rp.data(), ci.data(), mb, kb, pair_rows, pair_ptr, units);
  const size_t npairs = pair_ptr.empty() ? 0 : pair_ptr.size() - 1;
  std::printf("%.17g\n%zu\n", saving, npairs);
  for (size_t p = 0; p < npairs; ++p)
    std::printf("%d %d %d %d\n", pair_rows[2 * p], pair_rows[2 * p + 1], pair_ptr[p], pair_ptr[p + 1]);
  std::printf("%zu\n", units.size() / 4);
  for (size_t u = 0; u < units.size() / 4; ++u)
    std::printf("%d %d %d\n", units[4 * u], units[4 * u + 1], units[4 * u + 2]);
  return 0;
}
