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

template <typename T>
__device__ __forceinline__ uint4 load_vt_frag(const T* vrow, int kb0, int grp, int k_end);

// bf16: keys {kb0 + 4g + i} and {kb0 + 16 + 4g + i}, i < 4 (two 16-key blocks)
template <>
__device__ __forceinline__ uint4 load_vt_frag<bf16_t>(const bf16_t* vrow, int kb0, int grp,
                                                      int k_end) {
  const int ka = kb0 + 4 * grp, kb = kb0 + 16 + 4 * grp;
  uint2 lo = *reinterpret_cast<const uint2*>(vrow + ka);
  uint2 hi = *reinterpret_cast<const uint2*>(vrow + kb);
  uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
  // keys at or past k_end are zeroed with selects (a branch would wait for
  // each load on its own)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k0 = (i < 2 ? ka : kb) + 2 * (i % 2);
    w[i] &= k0 >= k_end ? 0u : (k0 + 1 >= k_end ? 0x0000ffffu : 0xffffffffu);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// fp32: keys {kb0 + 4g + i}, i < 4 (one 16-key block)
template <>
__device__ __forceinline__ uint4 load_vt_frag<float>(const float* vrow, int kb0, int grp,
                                                     int k_end) {
  const int ka = kb0 + 4 * grp;
  const uint4 v = *reinterpret_cast<const uint4*>(vrow + ka);
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

template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnArgs p) {
  using MM = Mma<T>;
  constexpr int E = MM::E;
  constexpr int KSTEP = MM::KSTEP;
  constexpr int NF = DH / KSTEP;    // Q^T fragments along head_dim
  constexpr int ND = DH / 16;       // O^T row blocks
  constexpr int NBLK = KSTEP / 16;  // 16-key S^T blocks per P^T fragment
  constexpr int PW = ND * kWave * 4 + 32;  // floats of one wave's partial
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
  const int qr0 = (qg * 4 + wave) * 16;
  const bool active = qr0 < R;
  const int len = p.n_valid[b] + p.T;
  const int k_begin = s * p.kc_len;
  const int k_end = min(k_begin + p.kc_len, len);

  const T* Kb = static_cast<const T*>(p.kcache) + static_cast<size_t>(b * p.Hkv + g) * p.S_max * DH;
  const T* Vb = static_cast<const T*>(p.vtcache) + static_cast<size_t>(b * p.Hkv + g) * DH * p.S_max;

  const int myq = qr0 + lane % 16;
  const bool qvalid = myq < R;
  const int hh = qvalid ? myq / p.T : 0;
  const int tt = qvalid ? myq % p.T : 0;

  uint4 qf[NF];
  {
    const T* qrow = static_cast<const T*>(p.q) + static_cast<size_t>(b * p.T + tt) * p.ldq +
                    (g * G + hh) * DH + E * grp;
#pragma unroll
    for (int kf = 0; kf < NF; ++kf)
      qf[kf] = *reinterpret_cast<const uint4*>(qrow + kf * KSTEP);  // rows past R: a valid row, unused
  }

  f32x4 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  if (active) {
    for (int kb0 = k_begin; kb0 < k_end; kb0 += KSTEP) {
      f32x4 st[NBLK];
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        st[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
        // keys past the split read its last key; their scores are masked below
        const int key = min(kb0 + 16 * blk + lane % 16, k_end - 1);
        const T* krow = Kb + static_cast<size_t>(key) * DH + E * grp;
#pragma unroll
        for (int kf = 0; kf < NF; ++kf) {
          const uint4 kfr = *reinterpret_cast<const uint4*>(krow + kf * KSTEP);
          st[blk] = MM::mma(kfr, qf[kf], st[blk]);
        }
      }
      // st[blk][i] = S^T[key kb0 + 16 blk + 4 grp + i][query lane % 16]
      float sv[NBLK * 4];
      float cmax = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + 16 * blk + 4 * grp + i;
          const float x = key < k_end ? st[blk][i] * p.scale_log2 : -INFINITY;
          sv[blk * 4 + i] = x;
          cmax = fmaxf(cmax, x);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, kWave));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, kWave));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = exp2f(m_run - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < NBLK * 4; ++i) {
        sv[i] = exp2f(sv[i] - m_new);
        psum += sv[i];
      }
      psum += __shfl_xor(psum, 16, kWave);
      psum += __shfl_xor(psum, 32, kWave);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const uint4 pf = pack_frag<T>(sv);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        acc[d] *= alpha;
        const T* vrow = Vb + static_cast<size_t>(16 * d + lane % 16) * p.S_max;
        const uint4 vf = load_vt_frag<T>(vrow, kb0, grp, k_end);
        acc[d] = MM::mma(vf, pf, acc[d]);
      }
    }
  }
  // acc[d][i] = O^T[dim 16 d + 4 grp + i][query lane % 16] (unnormalised)

  if (p.nsplit > 1) {
    float* part = p.partial + (static_cast<size_t>(item) * p.nsplit + s) * 4 * PW;
    float* mine = part + wave * PW;
    if (active) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
        st_dev4(reinterpret_cast<f32x4*>(mine + (d * kWave + lane) * 4), acc[d]);
      if (grp == 0) {
        st_dev(mine + ND * kWave * 4 + lane, m_run);
        st_dev(mine + ND * kWave * 4 + 16 + lane, l_run);
      }
    }
    if (!arrive_last(p.counters + item, p.nsplit, &s_flag)) return;
    if (active) {
      float mx = -INFINITY;
      for (int s2 = 0; s2 < p.nsplit; ++s2) {
        const float* ps = p.partial + (static_cast<size_t>(item) * p.nsplit + s2) * 4 * PW + wave * PW;
        mx = fmaxf(mx, ld_dev(ps + ND * kWave * 4 + lane % 16));
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run = 0.0f;
      for (int s2 = 0; s2 < p.nsplit; ++s2) {
        const float* ps = p.partial + (static_cast<size_t>(item) * p.nsplit + s2) * 4 * PW + wave * PW;
        const float ms = ld_dev(ps + ND * kWave * 4 + lane % 16);
        if (ms == -INFINITY) continue;
        const float w = exp2f(ms - mx);
        l_run += w * ld_dev(ps + ND * kWave * 4 + 16 + lane % 16);
#pragma unroll
        for (int d = 0; d < ND; ++d)
          acc[d] += w * ld_dev4(reinterpret_cast<const f32x4*>(ps + (d * kWave + lane) * 4));
      }
    }
  }

  if (active && qvalid) {
    const float inv = 1.0f / l_run;
    T* orow = static_cast<T*>(p.o) + static_cast<size_t>(b * p.T + tt) * p.ldo + (g * G + hh) * DH;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      float v[4] = {acc[d][0] * inv, acc[d][1] * inv, acc[d][2] * inv, acc[d][3] * inv};
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

size_t attention_partial_floats(int dh, int items, int nsplit) {
  const size_t pw = static_cast<size_t>(dh / 16) * kWave * 4 + 32;
  return static_cast<size_t>(items) * nsplit * 4 * pw;
}

hipError_t launch_attention(Dt dt, const AttnArgs& a, hipStream_t s) {
  const int items = a.batch * a.Hkv * a.n_qg;
  const int blocks = kXcds * a.nsplit * ((items + kXcds - 1) / kXcds);
  if (dt == DT_BF16) return launch_dh<bf16_t>(a, blocks, s);
  return launch_dh<float>(a, blocks, s);
}

}  // namespace ae
