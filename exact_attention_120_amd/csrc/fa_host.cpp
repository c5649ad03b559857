// fa_host.cpp -- host-side grid arithmetic of the forward launch (no device
// code): grid sizes for the C-ABI's size checks, the split count the library
// picks for split-KV and its choice of the key-split kernel. Kept apart from
// the kernels so that the C-ABI layer can also be built for the host alone
// (the sanitizer build of the ABI tests).
#include "fa_internal.hpp"

namespace fa {

long long fwd_grid_size(int B, int H, int N) {
  return (long long)B * H * ((N + kFwdRowsKeySplitMin - 1) / kFwdRowsKeySplitMin);
}

int fwd_rows_per_workgroup(int dtype) { return dtype == 0 ? kFwdRowsF32 : kFwdRows16; }

int fwd_auto_splits(int B, int H, int N, int dtype) {
  constexpr int kCUs = 256;
  const int bm = fwd_rows_per_workgroup(dtype);
  const long long wgs = (long long)B * H * ((N + bm - 1) / bm);
  const int nkt = (N + kFwdKeyTile - 1) / kFwdKeyTile;
  int s = 1;
  while (s < 16 && wgs * s < kCUs && nkt / (2 * s) >= 4) s *= 2;
  return s;
}

bool fwd_auto_key_split(int B, int H, int N, int d, int dtype, int causal) {
  constexpr int kCUs = 256;
  if (dtype == 0 || (d != 64 && d != 128)) return false;
  const long long wgs = (long long)B * H * ((N + kFwdRows16 - 1) / kFwdRows16);
  // Under the causal rule one full round of row tiles is still uneven (the
  // last tile of a head sees every key, the first a quarter of a tile's
  // worth or less), so the key split also wins at exactly one round.
  return causal ? wgs <= kCUs : wgs < kCUs;
}

}  // namespace fa
