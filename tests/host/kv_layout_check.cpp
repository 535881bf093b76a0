// Host check of the key-block K / V cache layout (KvLayout in ae_device.h):
// for bf16 and fp32 and head sizes 64, 128, 256,
//  * k_off and v_off are bijections of (key, column) onto the cache of one
//    (request, head) and keep each key inside its own key block;
//  * the K fragment of tile blk, dims kf * KSTEP.. holds, in lane (r, g),
//    element e: K[block key key_of(blk, r)][kf * KSTEP + E g + e];
//  * the 16 x 16 S^T tile puts rows 4 g .. 4 g + 3 in lane group g, and those
//    rows of the NBLK tiles are the keys E g .. E g + E - 1 in order;
//  * the V fragment fd holds, in lane (r, g), element e: V[key E g + e][16 fd + r].
// Prints the number of violations; exit status 0 when there are none.
#include "ae_device.h"

#include <cstdio>
#include <vector>

using namespace ae;

template <typename T>
static int check(int dh, int S) {
  using L = KvLayout<T>;
  const int E = L::E, KB = L::KB, NF = dh / KB, NBLK = L::NBLK;
  std::vector<int> hk(static_cast<size_t>(S) * dh, 0), hv(static_cast<size_t>(S) * dh, 0);
  int bad = 0;
  for (int key = 0; key < S; ++key)
    for (int c = 0; c < dh; ++c) {
      const size_t a = L::k_off(key, c, dh), b = L::v_off(key, c, dh);
      if (a >= hk.size() || b >= hv.size()) {
        ++bad;
        continue;
      }
      ++hk[a];
      ++hv[b];
      if (a / L::block_elems(dh) != static_cast<size_t>(key / KB)) ++bad;
      if (b / L::block_elems(dh) != static_cast<size_t>(key / KB)) ++bad;
    }
  for (size_t i = 0; i < hk.size(); ++i) bad += (hk[i] != 1) + (hv[i] != 1);
  for (int j = 0; j < S / KB; ++j)
    for (int blk = 0; blk < NBLK; ++blk)
      for (int kf = 0; kf < NF; ++kf)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < E; ++e) {
            const int r = l % 16, g = l / 16;
            const size_t want = (static_cast<size_t>(j * NBLK * NF + blk * NF + kf) * 64 + l) * E + e;
            if (L::k_off(j * KB + L::key_of(blk, r), kf * KB + E * g + e, dh) != want) ++bad;
          }
  for (int g = 0; g < 4; ++g)
    for (int blk = 0; blk < NBLK; ++blk)
      for (int i = 0; i < 4; ++i)
        if (L::key_of(blk, 4 * g + i) != E * g + 4 * blk + i) ++bad;
  for (int j = 0; j < S / KB; ++j)
    for (int fd = 0; fd < dh / 16; ++fd)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < E; ++e) {
          const int r = l % 16, g = l / 16;
          const size_t want = (static_cast<size_t>(j * (dh / 16) + fd) * 64 + l) * E + e;
          if (L::v_off(j * KB + E * g + e, 16 * fd + r, dh) != want) ++bad;
        }
  return bad;
}

int main() {
  int bad = 0;
  for (int dh : {64, 128, 256}) {
    bad += check<bf16_t>(dh, 128);
    bad += check<float>(dh, 128);
  }
  std::printf("kv layout violations: %d\n", bad);
  return bad != 0;
}
