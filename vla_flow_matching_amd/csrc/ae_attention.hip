// Attention of the action-chunk queries over [visible prefix K/V | the action
// tokens' own K/V] (LoongForge Pi0.5 blog, section 3: actions see every valid
// prefix token and each other; padding and empty camera slots are invisible;
// the KV head is broadcast to its query heads inside the kernel).
//
// The prefix was compacted at ingest (only visible rows were copied, in
// order), and the QKV epilogue appends the T action rows right after them, so
// the keys of request b are the contiguous rows [0, n_valid[b] + T) of its
// cache: masked rows are never read, and there is no per-element mask except
// the ragged tail of the last key block.  The DiT-style block (MolmoBot PR
// Part 2) runs the same kernel twice with other key ranges: its attn1 over a
// cache of the action rows alone (n_valid 0), its attn2 over the prefix alone
// (no action rows appended; with no visible row the output is zero).
//
// One wave owns 16 query rows of one KV group (rows = (query head in group,
// action token) pairs; all Hq/Hkv heads of a group share the keys).  Per key
// block it forms S^T = K . Q^T on the MFMA units, so each lane ends up owning
// one query's column: the online-softmax max/sum need only two cross-lane
// steps, and P^T feeds the O^T = V^T . P^T product straight from registers
// (V is kept transposed in the cache for that).  Keys are split across
// workgroups; the last workgroup of a query group merges the partial
// (max, sum, O) triples in split order, so results are reproducible.
#include "ae_device.h"
#include "ae_kernels.h"

namespace ae {

namespace {

constexpr int kThreads = 512;  // 8 waves: 4 row groups x 2 key halves
constexpr int kRowWaves = 4;
constexpr int kXcds = 8;
constexpr int kQB = 1;  // 16-row query blocks per wave
constexpr int kMergeBatch = 2;  // key splits merged per round of loads
constexpr int kSlots = 2;       // LDS slots of one step (two key blocks) each
constexpr int kManyItems = 32;     // items from which two key splits suffice
constexpr int kFewItemSplits = 8;  // key splits per item at most below that

template <typename T>
__device__ __forceinline__ void store4(T* dst, const float* v);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* dst, const float* v) {
  uint2 w;
  w.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
  w.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
  *reinterpret_cast<uint2*>(dst) = w;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, const float* v) {
  *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}

// Key blocks (KSTEP keys) in LDS, in the cache's fragment order (the
// key-block layout): NBLK * NF K fragments (S^T = K Q^T operands), then ND
// V^T fragments (O^T = V^T P^T operands), 1 KiB each, each a contiguous run
// of the cache.  A step is two consecutive blocks; the eight waves copy an
// eighth of its fragments each.  Keys of the last block past k_end are
// copied as they are: their scores are masked, and the cache holds finite
// values there (zeros or another split's keys), so their zero P contributes
// nothing.
template <typename T, int DH>
struct KvBlock {
  using MM = Mma<T>;
  using LY = KvLayout<T>;
  static constexpr int E = MM::E, KSTEP = MM::KSTEP;
  static constexpr int NF = DH / KSTEP, ND = DH / 16, NBLK = KSTEP / 16;
  static constexpr int NK = NBLK * NF, FPB = NK + ND;
  static_assert(FPB % 8 == 0 && NK % 4 == 0, "a step's fragments split evenly over 8 waves");

  // Kb / Vb: the (request, head)'s K and V caches; kb0: the step's first
  // key; nb: its blocks (1 or 2); lds: the LDS byte address of its slot;
  // wave: this wave's index (scalar); lane16 = 16 * lane
  static __device__ __forceinline__ void issue_step(const T* Kb, const T* Vb, int kb0, int nb, uint32_t lds,
                                                    int wave, uint32_t lane16) {
#pragma unroll
    for (int j = 0; j < 2 * FPB / 8; ++j) {
      const int x = 8 * j + wave, hb = x / FPB, f = x % FPB;
      if (hb >= nb) break;  // (x grows with j: the rest belongs to the absent block too)
      const size_t blk0 = static_cast<size_t>(kb0 / KSTEP + hb) * LY::block_elems(DH);
      const T* src = f < NK ? Kb + blk0 + f * kWave * E : Vb + blk0 + (f - NK) * kWave * E;
      dma_frag(src, lds + static_cast<uint32_t>(x * kWave * 16), lane16);
    }
  }
};

// One staged key block (KSTEP keys at kb0; fr = the block's LDS fragments
// + lane) against the wave's kQB query blocks: S^T = K Q^T on the MFMA units,
// the online softmax per query column, O^T += V^T P^T.
template <typename T, int DH, int QB>
__device__ __forceinline__ void attn_block(const uint4* fr, int kb0, int k_end, float scale_log2,
                                           const uint4 (&qf)[QB][DH / Mma<T>::KSTEP],
                                           f32x4 (&acc)[QB][DH / 16], float (&m_run)[QB], float (&l_run)[QB]) {
  using KV = KvBlock<T, DH>;
  using MM = Mma<T>;
  constexpr int KSTEP = KV::KSTEP, NF = KV::NF, ND = KV::ND, NBLK = KV::NBLK, NK = KV::NK;
  const int grp = (threadIdx.x % kWave) / 16;
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    f32x4 st[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      st[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kf = 0; kf < NF; ++kf) st[blk] = MM::mma(fr[(blk * NF + kf) * kWave], qf[c][kf], st[blk]);
    }
    // st[blk][i] = S^T[key kb0 + key_of(blk, 4 grp + i)][query lane % 16]: the
    // lane's keys kb0 + E grp .. in order
    float sv[NBLK * 4];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[blk * 4 + i] = st[blk][i];
    if (kb0 + KSTEP > k_end) {  // ragged last block (uniform branch)
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb0 + KvLayout<T>::key_of(blk, 4 * grp + i) >= k_end) sv[blk * 4 + i] = -INFINITY;
    }
    float cmax = sv[0];
#pragma unroll
    for (int i = 1; i < NBLK * 4; ++i) cmax = fmaxf(cmax, sv[i]);
    cmax = xor16_max(cmax);
    cmax = xor32_max(cmax) * scale_log2;
    if (!__all(cmax <= m_run[c] + kSoftmaxSlack)) {  // move the reference max
      const float m_new = fmaxf(m_run[c], cmax);
      const float alpha = exp2_hw(m_run[c] - m_new);
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[c][d] *= alpha;
      l_run[c] *= alpha;
      m_run[c] = m_new;
    }
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < NBLK * 4; ++i) {
      sv[i] = exp2_hw(fmaf(sv[i], scale_log2, -m_run[c]));
      psum += sv[i];
    }
    l_run[c] += psum;  // this lane's keys only: summed over the lane groups after the loop
    const uint4 pf = pack_frag<T>(sv);
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[c][d] = MM::mma(fr[(NK + d) * kWave], pf, acc[c][d]);
  }
}

// One workgroup = 4 row groups x kQB query blocks of 16 rows of one (request,
// KV group), over one split of the keys, with two waves per row group that
// take alternate key blocks (two independent waves per SIMD hide each
// other's softmax and LDS latency).  Key blocks are copied straight into LDS
// slots shared by the waves, one step of two blocks ahead, so every K/V byte
// crosses from L2 once per workgroup.
template <typename T, int DH>
__global__ __launch_bounds__(kThreads, 1) void attention_kernel(AttnArgs p) {
  using KV = KvBlock<T, DH>;
  using MM = Mma<T>;
  constexpr int E = KV::E, KSTEP = KV::KSTEP, NF = KV::NF, ND = KV::ND, NBLK = KV::NBLK;
  constexpr int NK = KV::NK, FPB = KV::FPB;
  constexpr int PW = ND * kWave * 4 + 32;  // floats of one query block's partial
  __shared__ uint4 s_kv[kSlots][2 * FPB * kWave];
  __shared__ int s_flag;

  const int G = p.Hq / p.Hkv;
  const int R = p.T * G;
  const int n_items = p.batch * p.Hkv * p.n_qg;
  // XCD x (= block index mod 8) runs the contiguous range [x C, x C + C) of
  // the units ordered by (item, split), so the query groups of a request
  // share one L2 and the splits of an item one XCD.
  const int n_units = n_items * p.nsplit, C = (n_units + kXcds - 1) / kXcds;
  if (static_cast<int>(blockIdx.x) >= kXcds * C) {  // a weight-prefetch workgroup
    prefetch_ranges<kThreads, 32>(p.pf, p.pf_n4, 4, blockIdx.x - kXcds * C, p.pf_blocks,
                                  static_cast<uint32_t>(reinterpret_cast<size_t>((lds_void_t*)(&s_kv[0][0]))));
    return;
  }
  const int li = blockIdx.x / kXcds, u = (blockIdx.x % kXcds) * C + li;
  if (li >= C || u >= n_units) return;
  const int s = u % p.nsplit;
  const int item = u / p.nsplit;
  const int qg = item % p.n_qg;
  const int bg = item / p.n_qg;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;

  const int wave = threadIdx.x / kWave, rg = wave % kRowWaves, kh = wave / kRowWaves;
  const int lane = threadIdx.x % kWave;
  const int grp = lane / 16;
  const int len = p.n_valid[b] + p.n_act;
  // the request's own keys spread evenly over the splits, in whole key
  // blocks (the plan's kc_len covers the bucket's largest request: a
  // request with fewer visible keys gets shorter splits, not empty ones)
  const int kc = min(p.kc_len, ((len + p.nsplit - 1) / p.nsplit + KSTEP - 1) / KSTEP * KSTEP);
  const int k_begin = s * kc;
  const int k_end = min(k_begin + kc, len);
  const int n_blk = k_end > k_begin ? (k_end - k_begin + KSTEP - 1) / KSTEP : 0;

  const T* Kb = static_cast<const T*>(p.kcache) + static_cast<size_t>(b * p.Hkv + g) * p.S_max * DH;
  const T* Vb = static_cast<const T*>(p.vtcache) + static_cast<size_t>(b * p.Hkv + g) * p.S_max * DH;

  // query rows of this wave's row group: blocks (qg * 4 + rg) * kQB + c, 16
  // rows each (both key halves hold the same rows)
  uint4 qf[kQB][NF];
  int hh[kQB], tt[kQB];
  bool qvalid[kQB];
#pragma unroll
  for (int c = 0; c < kQB; ++c) {
    const int myq = ((qg * 4 + rg) * kQB + c) * 16 + lane % 16;
    qvalid[c] = myq < R;
    const int q = min(myq, R - 1);  // rows past R read a valid row, never stored
    hh[c] = q / p.T;
    tt[c] = q % p.T;
    const T* qrow = static_cast<const T*>(p.q) + static_cast<size_t>(b * p.T + tt[c]) * p.ldq +
                    (g * G + hh[c]) * DH + E * grp;
#pragma unroll
    for (int kf = 0; kf < NF; ++kf) qf[c][kf] = *reinterpret_cast<const uint4*>(qrow + kf * KSTEP);
  }

  f32x4 acc[kQB][ND];
  float m_run[kQB], l_run[kQB];
#pragma unroll
  for (int c = 0; c < kQB; ++c) {
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[c][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[c] = -INFINITY;
    l_run[c] = 0.0f;
  }

  // Steps of two key blocks: the waves of key half kh take block 2 t + kh of
  // step t, so each SIMD runs two independent waves.  Steps stream through
  // kSlots LDS slots, copied one step ahead of the one being multiplied.
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_void_t*)(&s_kv[0][0])));
  constexpr uint32_t kSlotBytes = 2 * FPB * kWave * 16;
  const uint32_t lane16 = 16u * lane;
  const int n_steps = (n_blk + 1) / 2;
  if (n_steps > 0) KV::issue_step(Kb, Vb, k_begin, min(2, n_blk), lds0, swave, lane16);
  for (int t = 0; t < n_steps; ++t) {
    wait_vm<0>();     // this wave's copies of step t landed
    __syncthreads();  // every wave's have; step t - 1's slot is free
    if (t + 1 < n_steps)
      KV::issue_step(Kb, Vb, k_begin + 2 * (t + 1) * KSTEP, min(2, n_blk - 2 * (t + 1)),
                     lds0 + ((t + 1) % kSlots) * kSlotBytes, swave, lane16);
    const int bi = 2 * t + kh;
    if (bi < n_blk)
      attn_block<T, DH, kQB>(s_kv[t % kSlots] + kh * FPB * kWave + lane, k_begin + bi * KSTEP, k_end,
                             p.scale_log2, qf, acc, m_run, l_run);
  }
  // acc[c][d][i] = O^T[dim 16 d + 4 grp + i][query lane % 16 of block c] (unnormalised)
#pragma unroll
  for (int c = 0; c < kQB; ++c) l_run[c] = xor32_sum(xor16_sum(l_run[c]));

  // Key half 1 hands its (O^T, m, l) to key half 0 of the same rows through
  // LDS (the slots are free once every wave is past the loop); half 0
  // combines them, and from here on only half 0 carries the rows.
  __syncthreads();
  {
    uint4* xo = &s_kv[0][0] + rg * (kQB * ND + 1) * kWave;
    if (kh == 1) {
#pragma unroll
      for (int c = 0; c < kQB; ++c)
#pragma unroll
        for (int d = 0; d < ND; ++d) xo[(c * ND + d) * kWave + lane] = __builtin_bit_cast(uint4, acc[c][d]);
      xo[kQB * ND * kWave + lane] =
          make_uint4(__float_as_uint(m_run[0]), __float_as_uint(l_run[0]),
                     __float_as_uint(kQB > 1 ? m_run[kQB - 1] : 0.0f), __float_as_uint(kQB > 1 ? l_run[kQB - 1] : 0.0f));
    }
    __syncthreads();
    if (kh == 0) {
      const uint4 ml = xo[kQB * ND * kWave + lane];
#pragma unroll
      for (int c = 0; c < kQB; ++c) {
        const float m1 = __uint_as_float(c == 0 ? ml.x : ml.z), l1 = __uint_as_float(c == 0 ? ml.y : ml.w);
        const float m_new = fmaxf(m_run[c], m1);
        if (m_new != -INFINITY) {  // (both halves empty: nothing to combine)
          const float a0 = exp2_hw(m_run[c] - m_new), a1 = exp2_hw(m1 - m_new);
#pragma unroll
          for (int d = 0; d < ND; ++d)
            acc[c][d] = acc[c][d] * a0 + a1 * __builtin_bit_cast(f32x4, xo[(c * ND + d) * kWave + lane]);
          l_run[c] = l_run[c] * a0 + l1 * a1;
          m_run[c] = m_new;
        }
      }
    }
  }

  if (p.nsplit > 1) {
    // publish every query block's (O^T, m, l), then the last split of the
    // item merges them in split order
    const size_t per_split = static_cast<size_t>(4 * kQB) * PW;
    float* part = p.partial + static_cast<size_t>(item) * p.nsplit * per_split;
    const Coh cp(part);
#pragma unroll
    for (int c = 0; c < kQB; ++c) {
      if (kh != 0) break;
      const uint32_t wb = 4u * static_cast<uint32_t>(s * per_split + (rg * kQB + c) * PW);
#pragma unroll
      for (int d = 0; d < ND; ++d)
        cp.st16(wb + 16u * (d * kWave + lane),
                make_uint4(__float_as_uint(acc[c][d][0]), __float_as_uint(acc[c][d][1]),
                           __float_as_uint(acc[c][d][2]), __float_as_uint(acc[c][d][3])));
      if (grp == 0) {
        cp.stf(wb + 4u * (ND * kWave * 4 + lane), m_run[c]);
        cp.stf(wb + 4u * (ND * kWave * 4 + 16 + lane), l_run[c]);
      }
    }
    if (!arrive_last(p.counters + item, p.nsplit, &s_flag)) return;
#pragma unroll
    for (int c = 0; c < kQB; ++c) {
      if (kh != 0) break;
      float mx = -INFINITY, lsum = 0.0f;
      f32x4 o[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < p.nsplit; s0 += kMergeBatch) {
        // every split of the batch requested at once (clamped index)
        float ms[kMergeBatch], ls[kMergeBatch];
        uint4 av[kMergeBatch][ND];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const int s2 = min(s0 + j, p.nsplit - 1);
          const uint32_t wb = 4u * static_cast<uint32_t>(s2 * per_split + (rg * kQB + c) * PW);
          ms[j] = cp.ldf(wb + 4u * (ND * kWave * 4 + lane % 16));
          ls[j] = cp.ldf(wb + 4u * (ND * kWave * 4 + 16 + lane % 16));
#pragma unroll
          for (int d = 0; d < ND; ++d) av[j][d] = cp.ld16(wb + 16u * (d * kWave + lane));
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          if (s0 + j >= p.nsplit || ms[j] == -INFINITY) continue;  // repeat or empty split
          const float m_new = fmaxf(mx, ms[j]);
          const float a_old = exp2_hw(mx - m_new), a_new = exp2_hw(ms[j] - m_new);
          lsum = lsum * a_old + ls[j] * a_new;
#pragma unroll
          for (int d = 0; d < ND; ++d)
            o[d] = o[d] * a_old + a_new * f32x4{__uint_as_float(av[j][d].x), __uint_as_float(av[j][d].y),
                                                __uint_as_float(av[j][d].z), __uint_as_float(av[j][d].w)};
          mx = m_new;
        }
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[c][d] = o[d];
      l_run[c] = lsum;
    }
  }

#pragma unroll
  for (int c = 0; c < kQB; ++c) {
    if (kh != 0 || !qvalid[c]) continue;
    const float inv = l_run[c] > 0.0f ? 1.0f / l_run[c] : 0.0f;  // (no key: zeros)
    T* orow = static_cast<T*>(p.o) + static_cast<size_t>(b * p.T + tt[c]) * p.ldo + (g * G + hh[c]) * DH;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      float v[4] = {acc[c][d][0] * inv, acc[c][d][1] * inv, acc[c][d][2] * inv, acc[c][d][3] * inv};
      store4<T>(orow + 16 * d + 4 * grp, v);
    }
  }
}

template <typename T>
hipError_t launch_dh(const AttnArgs& a, int blocks, hipStream_t s) {
  dim3 grid(blocks), block(kThreads);
  switch (a.dh) {
    case 64: hipLaunchKernelGGL((attention_kernel<T, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((attention_kernel<T, 128>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((attention_kernel<T, 256>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t attention_partial_floats(int dh, int items, int nsplit, int rows_per_item) {
  const size_t pw = static_cast<size_t>(dh / 16) * kWave * 4 + 32;
  return static_cast<size_t>(items) * nsplit * (rows_per_item / 16) * pw;
}

int attention_rows_per_item() { return 4 * kQB * 16; }

// Key splits per item at most: each split writes, and the last one re-reads,
// a full fp32 O^T per query row, and that merge runs in one workgroup per
// item, so with items enough to fill the GPU few long splits beat many short
// ones; with few items (one or two requests) the key loop of each item is
// the critical path, and more splits shorten it.
int attention_max_splits(int items) {
  return items >= kManyItems ? 2 : kFewItemSplits;
}

hipError_t launch_attention(Dt dt, const AttnArgs& a, hipStream_t s) {
  const int items = a.batch * a.Hkv * a.n_qg;
  const int blocks = kXcds * ((items * a.nsplit + kXcds - 1) / kXcds) + a.pf_blocks;
  if (dt == DT_BF16) return launch_dh<bf16_t>(a, blocks, s);
  return launch_dh<float>(a, blocks, s);
}

}  // namespace ae
