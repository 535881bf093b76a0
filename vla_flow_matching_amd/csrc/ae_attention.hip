// Attention of the action-chunk queries over [visible prefix K/V | the action
// tokens' own K/V] (LoongForge Pi0.5 blog, section 3: actions see every valid
// prefix token and each other; padding and empty camera slots are invisible;
// the KV head is broadcast to its query heads inside the kernel).
//
// The prefix was compacted at ingest (only visible rows were copied, in
// order), and the QKV epilogue appends the T action rows right after them, so
// the keys of request b are the contiguous rows [0, n_valid[b] + T) of its
// cache: masked rows are never read, and there is no per-element mask except
// the ragged tail of the last key block.
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

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kQB = 1;  // 16-row query blocks per wave
constexpr int kMergeBatch = 2;  // key splits merged per round of loads

template <typename T>
__device__ __forceinline__ uint4 load_vt_frag(const T* vrow, int kb0, int grp, int k_end, bool tail);

// bf16: keys {kb0 + 4g + i} and {kb0 + 16 + 4g + i}, i < 4 (two 16-key blocks)
// `tail` (uniform): the block reaches past k_end, whose keys are zeroed with
// selects (a branch would wait for each load on its own); full blocks skip
// the masking.
template <>
__device__ __forceinline__ uint4 load_vt_frag<bf16_t>(const bf16_t* vrow, int kb0, int grp,
                                                      int k_end, bool tail) {
  const int ka = kb0 + 4 * grp, kb = kb0 + 16 + 4 * grp;
  uint2 lo = *reinterpret_cast<const uint2*>(vrow + ka);
  uint2 hi = *reinterpret_cast<const uint2*>(vrow + kb);
  uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
  if (tail) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = (i < 2 ? ka : kb) + 2 * (i % 2);
      w[i] &= k0 >= k_end ? 0u : (k0 + 1 >= k_end ? 0x0000ffffu : 0xffffffffu);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// fp32: keys {kb0 + 4g + i}, i < 4 (one 16-key block)
template <>
__device__ __forceinline__ uint4 load_vt_frag<float>(const float* vrow, int kb0, int grp,
                                                     int k_end, bool tail) {
  const int ka = kb0 + 4 * grp;
  const uint4 v = *reinterpret_cast<const uint4*>(vrow + ka);
  if (!tail) return v;
  return make_uint4(v.x & (ka + 0 >= k_end ? 0u : 0xffffffffu), v.y & (ka + 1 >= k_end ? 0u : 0xffffffffu),
                    v.z & (ka + 2 >= k_end ? 0u : 0xffffffffu), v.w & (ka + 3 >= k_end ? 0u : 0xffffffffu));
}

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

// Stage one key block (KSTEP keys) into LDS in fragment order: NBLK * NF K
// fragments (S^T = K Q^T operands), then ND V^T fragments (O^T = V^T P^T
// operands), 1 KiB each; the four waves load a quarter each.  Keys past
// k_end read a clamped row (K: their scores are masked) or are zeroed (V^T).
template <typename T, int DH>
struct KvBlock {
  using MM = Mma<T>;
  static constexpr int E = MM::E, KSTEP = MM::KSTEP;
  static constexpr int NF = DH / KSTEP, ND = DH / 16, NBLK = KSTEP / 16;
  static constexpr int NK = NBLK * NF, FPB = NK + ND, PER_WAVE = FPB / 4;
  static_assert(FPB % 4 == 0 && NK % 4 == 0, "fragments split evenly over 4 waves");

  static __device__ __forceinline__ void load(const T* Kb, const T* Vb, int S_max, int kb0, int k_end,
                                              uint4 (&v)[PER_WAVE]) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, grp = lane / 16;
    const bool tail = kb0 + KSTEP > k_end;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int f = 4 * j + wave;
      if (j < NK / 4) {
        const int blk = f / NF, kf = f % NF;
        const int kr = min(kb0 + 16 * blk + lane % 16, k_end - 1);
        v[j] = *reinterpret_cast<const uint4*>(Kb + static_cast<size_t>(kr) * DH + kf * KSTEP + E * grp);
      } else {
        const int vr = 16 * (f - NK) + lane % 16;
        v[j] = load_vt_frag<T>(Vb + static_cast<size_t>(vr) * S_max, kb0, grp, k_end, tail);
      }
    }
  }
  static __device__ __forceinline__ void store(uint4* dst, const uint4 (&v)[PER_WAVE]) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) dst[(4 * j + wave) * kWave + lane] = v[j];
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
    // st[blk][i] = S^T[key kb0 + 16 blk + 4 grp + i][query lane % 16]
    float sv[NBLK * 4];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[blk * 4 + i] = st[blk][i] * scale_log2;
    if (kb0 + KSTEP > k_end) {  // ragged last block (uniform branch)
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb0 + 16 * blk + 4 * grp + i >= k_end) sv[blk * 4 + i] = -INFINITY;
    }
    float cmax = sv[0];
#pragma unroll
    for (int i = 1; i < NBLK * 4; ++i) cmax = fmaxf(cmax, sv[i]);
    cmax = xor16_max(cmax);
    cmax = xor32_max(cmax);
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
      sv[i] = exp2_hw(sv[i] - m_run[c]);
      psum += sv[i];
    }
    psum = xor16_sum(psum);
    psum = xor32_sum(psum);
    l_run[c] += psum;
    const uint4 pf = pack_frag<T>(sv);
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[c][d] = MM::mma(fr[(NK + d) * kWave], pf, acc[c][d]);
  }
}

// One workgroup = 4 waves x kQB query blocks of 16 rows of one (request, KV
// group), over one split of the keys.  Key blocks are staged through two LDS
// buffers shared by the waves (the next block's loads are in flight while
// the current one is multiplied), so every K/V byte crosses from L2 once per
// workgroup.
template <typename T, int DH>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(AttnArgs p) {
  using KV = KvBlock<T, DH>;
  using MM = Mma<T>;
  constexpr int E = KV::E, KSTEP = KV::KSTEP, NF = KV::NF, ND = KV::ND, NBLK = KV::NBLK;
  constexpr int NK = KV::NK, FPB = KV::FPB;
  constexpr int PW = ND * kWave * 4 + 32;  // floats of one query block's partial
  __shared__ uint4 s_kv[2][FPB * kWave];
  __shared__ int s_flag;

  const int G = p.Hq / p.Hkv;
  const int R = p.T * G;
  const int n_items = p.batch * p.Hkv * p.n_qg;
  const int bid = blockIdx.x;
  int idx = bid / kXcds;
  const int s = idx % p.nsplit;
  const int item = (idx / p.nsplit) * kXcds + bid % kXcds;
  if (item >= n_items) return;
  const int qg = item % p.n_qg;
  const int bg = item / p.n_qg;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int grp = lane / 16;
  const int len = p.n_valid[b] + p.T;
  const int k_begin = s * p.kc_len;
  const int k_end = min(k_begin + p.kc_len, len);
  const int n_blk = k_end > k_begin ? (k_end - k_begin + KSTEP - 1) / KSTEP : 0;

  const T* Kb = static_cast<const T*>(p.kcache) + static_cast<size_t>(b * p.Hkv + g) * p.S_max * DH;
  const T* Vb = static_cast<const T*>(p.vtcache) + static_cast<size_t>(b * p.Hkv + g) * DH * p.S_max;

  // query rows of this wave: blocks (qg * 4 + wave) * kQB + c, 16 rows each
  uint4 qf[kQB][NF];
  int hh[kQB], tt[kQB];
  bool qvalid[kQB];
#pragma unroll
  for (int c = 0; c < kQB; ++c) {
    const int myq = ((qg * 4 + wave) * kQB + c) * 16 + lane % 16;
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

  uint4 stage[KV::PER_WAVE];
  if (n_blk > 0) {
    KV::load(Kb, Vb, p.S_max, k_begin, k_end, stage);
    KV::store(s_kv[0], stage);
  }
  __syncthreads();
  for (int bi = 0; bi < n_blk; ++bi) {
    KV::load(Kb, Vb, p.S_max, k_begin + min(bi + 1, n_blk - 1) * KSTEP, k_end, stage);
    attn_block<T, DH, kQB>(s_kv[bi & 1] + lane, k_begin + bi * KSTEP, k_end, p.scale_log2, qf, acc, m_run,
                           l_run);
    KV::store(s_kv[(bi + 1) & 1], stage);
    __syncthreads();
  }
  // acc[c][d][i] = O^T[dim 16 d + 4 grp + i][query lane % 16 of block c] (unnormalised)

  if (p.nsplit > 1) {
    // publish every query block's (O^T, m, l), then the last split of the
    // item merges them in split order
    const size_t per_split = static_cast<size_t>(4 * kQB) * PW;
    float* part = p.partial + static_cast<size_t>(item) * p.nsplit * per_split;
    const Coh cp(part);
#pragma unroll
    for (int c = 0; c < kQB; ++c) {
      const uint32_t wb = 4u * static_cast<uint32_t>(s * per_split + (wave * kQB + c) * PW);
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
          const uint32_t wb = 4u * static_cast<uint32_t>(s2 * per_split + (wave * kQB + c) * PW);
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
    if (!qvalid[c]) continue;
    const float inv = 1.0f / l_run[c];
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
// item, so few long splits beat many short ones.
int attention_max_splits(int items) {
  (void)items;
  return 2;
}

hipError_t launch_attention(Dt dt, const AttnArgs& a, hipStream_t s) {
  const int items = a.batch * a.Hkv * a.n_qg;
  const int blocks = kXcds * a.nsplit * ((items + kXcds - 1) / kXcds);
  if (dt == DT_BF16) return launch_dh<bf16_t>(a, blocks, s);
  return launch_dh<float>(a, blocks, s);
}

}  // namespace ae
