// Projection GEMMs of the action expert: Y[M, N] = A[M, K] . W[K, N] on the
// 16x16 MFMA units, with the expert's element-wise work fused in.
//
// * Prologue PRO_ADARMS builds A on the fly from the fp32 residual h:
//   u = h * r_m * (1 + scale) + shift, r_m = 1/sqrt(mean_k h^2 + eps), the
//   adaRMS modulation of the LoongForge Pi0.5 blog (section 2), rounded to
//   the operand type.  The row sums of squares arrive as per-tile partials
//   written by whichever kernel last updated h.
// * Epilogues: EPI_QKV rotates q and k (rotate_half RoPE, blog section 2) and
//   scatters q to its buffer and k / v into the request's K / V^T cache rows
//   n_valid + t; EPI_GELU forms gelu_tanh(gate) * up from paired columns;
//   EPI_RESID applies the gated residual h += gate * y and emits the new
//   rows' partial sums of squares.
//
// Weights are pre-packed (at load) in MFMA fragment order so every wave
// streams its B operand as contiguous 1 KiB blocks straight into registers,
// with no LDS staging: at the small M of the denoise loop the weights are
// read once and the A operand is small.  Work is split over K (split-K) so
// that the batch-1 GEMMs still cover every CU; partials are reduced in a
// fixed order by the last-arriving workgroup of each tile, so results are
// bitwise reproducible.  The four waves of a workgroup split the K range
// further and are reduced through LDS.  All splits and m-tiles of one n-tile
// run on one XCD (workgroups are dealt to XCDs round-robin), so they share
// that XCD's L2 for the weight slice and the partials.
#include "ae_device.h"
#include "ae_kernels.h"

namespace ae {

namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct TileIdx {
  int nt, mt, s, tile;
  bool valid;
};

__device__ __forceinline__ TileIdx decode_block(int bid, int n_tiles, int m_tiles, int ksplit) {
  TileIdx t;
  int xcd = bid % kXcds;
  int idx = bid / kXcds;
  t.s = idx % ksplit;
  idx /= ksplit;
  t.mt = idx % m_tiles;
  idx /= m_tiles;
  t.nt = idx * kXcds + xcd;
  t.valid = t.nt < n_tiles;
  t.tile = t.nt * m_tiles + t.mt;
  return t;
}

template <typename T>
__device__ __forceinline__ uint4 load_a_plain(const T* A, int lda, int row, int M, int k) {
  if (row >= M) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(A + static_cast<size_t>(row) * lda + k);
}

template <typename T>
__device__ __forceinline__ uint4 load_a_adarms(const float* h, int ldh, int row, int M, int k,
                                               float r, const float* scale, const float* shift) {
  constexpr int E = Mma<T>::E;
  if (row >= M) return make_uint4(0, 0, 0, 0);
  float v[E];
  const float4* hp = reinterpret_cast<const float4*>(h + static_cast<size_t>(row) * ldh + k);
  const float4* sp = reinterpret_cast<const float4*>(scale + k);
  const float4* bp = reinterpret_cast<const float4*>(shift + k);
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
    float4 hv = hp[j], sv = sp[j], bv = bp[j];
    v[4 * j + 0] = hv.x * r * (1.0f + sv.x) + bv.x;
    v[4 * j + 1] = hv.y * r * (1.0f + sv.y) + bv.y;
    v[4 * j + 2] = hv.z * r * (1.0f + sv.z) + bv.z;
    v[4 * j + 3] = hv.w * r * (1.0f + sv.w) + bv.w;
  }
  return pack_frag<T>(v);
}

template <typename T, int PRO, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  using MM = Mma<T>;
  constexpr int E = MM::E;
  constexpr int KSTEP = MM::KSTEP;
  constexpr int MT = kTileM / 16;  // 4 row fragments
  constexpr int NB = kTileN / 16;  // 4 column fragments

  // cross-wave reduction (64 KiB), later reused for the finished tile
  __shared__ __attribute__((aligned(16))) char s_raw[4 * MT * NB * kWave * sizeof(f32x4)];
  auto s_red = reinterpret_cast<f32x4 (*)[MT * NB][kWave]>(s_raw);
  auto s_y = reinterpret_cast<float (*)[kTileN + 1]>(s_raw);
  static_assert(kTileM * (kTileN + 1) * sizeof(float) <= sizeof(s_raw), "tile fits");
  __shared__ float s_r[kTileM];
  __shared__ int s_flag;

  const TileIdx ti = decode_block(blockIdx.x, p.n_tiles, p.m_tiles, p.ksplit);
  if (!ti.valid) return;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int m0 = ti.mt * kTileM;
  const int rows = min(kTileM, p.M - m0);
  const int mtr = (rows + 15) / 16;

  if (PRO == PRO_ADARMS) {
    if (tid < rows) {
      float acc = 0.0f;
      for (int t = 0; t < p.ssq_tiles; ++t) acc += p.ssq[t * p.ldssq + m0 + tid];
      s_r[tid] = 1.0f / sqrtf(acc / static_cast<float>(p.K) + p.eps);
    }
    __syncthreads();
  }

  const int kf0 = static_cast<int>((static_cast<long long>(ti.s) * p.k_frags) / p.ksplit);
  const int kf1 = static_cast<int>((static_cast<long long>(ti.s + 1) * p.k_frags) / p.ksplit);

  f32x4 acc[MT][NB];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = lane % 16;
  const int acol = E * (lane / 16);
  float rr[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    int r = 16 * i + arow;
    rr[i] = (PRO == PRO_ADARMS && r < rows) ? s_r[r] : 0.0f;
  }
  const uint4* Wt = p.W + static_cast<size_t>(ti.nt) * NB * p.k_frags * kWave + lane;

  for (int kf = kf0 + wave; kf < kf1; kf += 4) {
    uint4 b[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = Wt[(static_cast<size_t>(j) * p.k_frags + kf) * kWave];
    const int k = kf * KSTEP + acol;
    uint4 a[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i < mtr) {
        int row = m0 + 16 * i + arow;
        if (PRO == PRO_ADARMS)
          a[i] = load_a_adarms<T>(static_cast<const float*>(p.A), p.lda, row, p.M, k, rr[i],
                                  p.scale, p.shift);
        else
          a[i] = load_a_plain<T>(static_cast<const T*>(p.A), p.lda, row, p.M, k);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (i < mtr) {
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = MM::mma(a[i], b[j], acc[i][j]);
      }
  }

  // reduce the four waves' K slices: thread (wave j, lane) ends up owning
  // column fragment j of every row fragment
#pragma unroll
  for (int i = 0; i < MT; ++i)
    if (i < mtr)
#pragma unroll
      for (int j = 0; j < NB; ++j) s_red[wave][i * NB + j][lane] = acc[i][j];
  __syncthreads();
  const int jc = wave;
  f32x4 v[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < mtr) {
#pragma unroll
      for (int w = 0; w < 4; ++w) v[i] += s_red[w][i * NB + jc][lane];
    }
  }
  __syncthreads();  // s_red is dead from here on; s_raw becomes s_y

  if (p.ksplit > 1) {
    f32x4* part = reinterpret_cast<f32x4*>(p.partial) +
                  static_cast<size_t>(ti.tile) * p.ksplit * (MT * NB * kWave);
    f32x4* mine = part + static_cast<size_t>(ti.s) * (MT * NB * kWave);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (i < mtr) st_dev4(&mine[(i * NB + jc) * kWave + lane], v[i]);
    if (!arrive_last(p.counters + ti.tile, p.ksplit, &s_flag)) return;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i < mtr) {
        f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < p.ksplit; ++s) {
          const f32x4* ps = part + static_cast<size_t>(s) * (MT * NB * kWave);
          tot += ld_dev4(&ps[(i * NB + jc) * kWave + lane]);
        }
        v[i] = tot;
      }
    }
  }

  // finished tile -> LDS
#pragma unroll
  for (int i = 0; i < MT; ++i)
    if (i < mtr)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_y[16 * i + 4 * (lane / 16) + e][16 * jc + lane % 16] = v[i][e];
  __syncthreads();

  if (EPI == EPI_RESID) {
    // one row per wave per step, 64 lanes = the tile's 64 columns
    for (int row = wave; row < rows; row += 4) {
      const int m = m0 + row;
      const int n = ti.nt * kTileN + lane;
      float* hp = p.h + static_cast<size_t>(m) * p.ldh + n;
      float hn = *hp + p.gate[n] * s_y[row][lane];
      *hp = hn;
      float sq = wave_sum(hn * hn);
      if (lane == 0) p.ssq_out[ti.nt * p.ldssq + m] = sq;
    }
  } else if (EPI == EPI_GELU) {
    T* out = static_cast<T*>(p.out);
    for (int idx = tid; idx < rows * 32; idx += kThreads) {
      const int row = idx / 32, c = idx % 32, pr = c / 16, jj = c % 16;
      const float g = s_y[row][32 * pr + jj];
      const float u = s_y[row][32 * pr + 16 + jj];
      const int f = (2 * ti.nt + pr) * 16 + jj;
      out[static_cast<size_t>(m0 + row) * p.ldo + f] = Elem<T>::from_f(gelu_tanh(g) * u);
    }
  } else {  // EPI_QKV
    const int pph = p.dh / 32;  // column pairs per head
    const int pq = p.Hq * pph, pk = p.Hkv * pph;
    const int half = p.dh / 2;
    T* qo = static_cast<T*>(p.q);
    T* kc = static_cast<T*>(p.kcache);
    T* vt = static_cast<T*>(p.vtcache);
    for (int idx = tid; idx < rows * 32; idx += kThreads) {
      const int row = idx / 32, c = idx % 32, pr = c / 16, jj = c % 16;
      const int P = 2 * ti.nt + pr;
      float a = s_y[row][32 * pr + jj];
      float b = s_y[row][32 * pr + 16 + jj];
      const int m = m0 + row;
      const int req = m / p.T, t = m % p.T;
      int seg, head, pi;
      if (P < pq) { seg = 0; head = P / pph; pi = P % pph; }
      else if (P < pq + pk) { seg = 1; head = (P - pq) / pph; pi = (P - pq) % pph; }
      else { seg = 2; head = (P - pq - pk) / pph; pi = (P - pq - pk) % pph; }
      const int j = 16 * pi + jj;
      if (seg < 2) {
        const size_t ti2 = (static_cast<size_t>(req) * p.T + t) * half + j;
        const float cs = p.rope_cos[ti2], sn = p.rope_sin[ti2];
        const float ra = a * cs - b * sn;
        const float rb = b * cs + a * sn;
        a = ra;
        b = rb;
      }
      if (seg == 0) {
        T* dst = qo + static_cast<size_t>(m) * p.ldq + head * p.dh;
        dst[j] = Elem<T>::from_f(a);
        dst[half + j] = Elem<T>::from_f(b);
      } else {
        const int key = p.n_valid[req] + t;
        const size_t base = static_cast<size_t>(req) * p.Hkv + head;
        using LY = KvLayout<T>;
        T* dst = (seg == 1 ? kc : vt) + base * p.S_max * p.dh;
        if (seg == 1) {
          dst[LY::k_off(key, j, p.dh)] = Elem<T>::from_f(a);
          dst[LY::k_off(key, half + j, p.dh)] = Elem<T>::from_f(b);
        } else {
          dst[LY::v_off(key, j, p.dh)] = Elem<T>::from_f(a);
          dst[LY::v_off(key, half + j, p.dh)] = Elem<T>::from_f(b);
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_t(Prologue pro, Epilogue epi, const GemmArgs& a, int blocks, hipStream_t s) {
  dim3 grid(blocks), block(kThreads);
#define AE_GEMM_CASE(P, EP)                                                       \
  if (pro == P && epi == EP) {                                                    \
    hipLaunchKernelGGL((gemm_kernel<T, P, EP>), grid, block, 0, s, a);            \
    return hipGetLastError();                                                     \
  }
  AE_GEMM_CASE(PRO_ADARMS, EPI_QKV)
  AE_GEMM_CASE(PRO_ADARMS, EPI_GELU)
  AE_GEMM_CASE(PRO_NONE, EPI_RESID)
  AE_GEMM_CASE(PRO_NONE, EPI_GELU)
  AE_GEMM_CASE(PRO_NONE, EPI_QKV)
  AE_GEMM_CASE(PRO_ADARMS, EPI_RESID)
#undef AE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int kstep_of(Dt dt) { return dt == DT_BF16 ? Mma<bf16_t>::KSTEP : Mma<float>::KSTEP; }

GemmPlan plan_gemm(Dt dt, int M, int N, int K, int target_blocks) {
  GemmPlan g;
  g.m_tiles = (M + kTileM - 1) / kTileM;
  g.n_tiles = N / kTileN;
  g.k_frags = K / kstep_of(dt);
  const int tiles = g.m_tiles * g.n_tiles;
  int s = (target_blocks + tiles - 1) / tiles;
  const int max_s = g.k_frags / 4 > 0 ? g.k_frags / 4 : 1;  // every wave gets a fragment
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  g.ksplit = s;
  const int nt_hi = (g.n_tiles + kXcds - 1) / kXcds;
  g.blocks = kXcds * g.ksplit * g.m_tiles * nt_hi;
  return g;
}

hipError_t launch_gemm(Dt dt, Prologue pro, Epilogue epi, const GemmArgs& a, int blocks,
                       hipStream_t s) {
  if (dt == DT_BF16) return launch_t<bf16_t>(pro, epi, a, blocks, s);
  return launch_t<float>(pro, epi, a, blocks, s);
}

// ---------------------------------------------------------------------------
// Weight packing: logical [K][N] row-major sources -> fragment order
// [N/16 column blocks][K/KSTEP k-fragments][64 lanes][16 bytes].
// ---------------------------------------------------------------------------

namespace {

template <typename T>
__global__ void pack_kernel(int mode, const T* s0, const T* s1, const T* s2, int K, int N,
                            int ld0, int ld1, int ld2, int Hq, int Hkv, int dh, uint4* dst,
                            int kvalid, int nvalid) {
  constexpr int E = Mma<T>::E;
  constexpr int KSTEP = Mma<T>::KSTEP;
  const int k_frags = K / KSTEP;
  const size_t total = static_cast<size_t>(N / 16) * k_frags * kWave;
  for (size_t g = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; g < total;
       g += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int lane = static_cast<int>(g % kWave);
    const size_t fr = g / kWave;
    const int kf = static_cast<int>(fr % k_frags);
    const int nb = static_cast<int>(fr / k_frags);
    const int pc = 16 * nb + lane % 16;
    const int k0 = kf * KSTEP + E * (lane / 16);
    const T* src;
    int ld, col;
    if (mode == PACK_PLAIN) {
      src = s0; ld = ld0; col = pc;
    } else {
      const int P = pc / 32, hf = (pc / 16) % 2, jj = pc % 16;
      if (mode == PACK_GU) {
        src = hf ? s1 : s0; ld = hf ? ld1 : ld0; col = 16 * P + jj;
      } else {
        const int pph = dh / 32, pq = Hq * pph, pk = Hkv * pph;
        int seg, head, pi;
        if (P < pq) { seg = 0; head = P / pph; pi = P % pph; }
        else if (P < pq + pk) { seg = 1; head = (P - pq) / pph; pi = (P - pq) % pph; }
        else { seg = 2; head = (P - pq - pk) / pph; pi = (P - pq - pk) % pph; }
        src = seg == 0 ? s0 : (seg == 1 ? s1 : s2);
        ld = seg == 0 ? ld0 : (seg == 1 ? ld1 : ld2);
        col = head * dh + hf * (dh / 2) + 16 * pi + jj;
      }
    }
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i)
      v[i] = (k0 + i < kvalid && col < nvalid) ? Elem<T>::to_f(src[static_cast<size_t>(k0 + i) * ld + col])
                                               : 0.0f;
    dst[g] = pack_frag<T>(v);
  }
}

// dst = fp32(src), or with cols > 0 the transpose of src [n / cols][cols]
template <typename T>
__global__ void to_f32_kernel(const T* src, float* dst, size_t n, int cols) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    if (cols > 0) {
      const size_t rows = n / cols, r = i / cols, c = i % cols;
      dst[c * rows + r] = Elem<T>::to_f(src[i]);
    } else {
      dst[i] = Elem<T>::to_f(src[i]);
    }
  }
}

}  // namespace

hipError_t launch_pack(Dt dt, PackMode mode, const void* s0, const void* s1, const void* s2,
                       int K, int N, int ld0, int ld1, int ld2, int Hq, int Hkv, int dh,
                       uint4* dst, hipStream_t s, int kvalid, int nvalid) {
  dim3 grid(1024), block(256);
  if (kvalid < 0) kvalid = K;
  if (nvalid < 0) nvalid = N;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(pack_kernel<bf16_t>, grid, block, 0, s, static_cast<int>(mode),
                       static_cast<const bf16_t*>(s0), static_cast<const bf16_t*>(s1),
                       static_cast<const bf16_t*>(s2), K, N, ld0, ld1, ld2, Hq, Hkv, dh, dst,
                       kvalid, nvalid);
  else
    hipLaunchKernelGGL(pack_kernel<float>, grid, block, 0, s, static_cast<int>(mode),
                       static_cast<const float*>(s0), static_cast<const float*>(s1),
                       static_cast<const float*>(s2), K, N, ld0, ld1, ld2, Hq, Hkv, dh, dst,
                       kvalid, nvalid);
  return hipGetLastError();
}

hipError_t launch_to_f32(Dt dt, const void* src, float* dst, size_t n, int transpose_cols,
                         hipStream_t s) {
  dim3 grid(256), block(256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(to_f32_kernel<bf16_t>, grid, block, 0, s, static_cast<const bf16_t*>(src),
                       dst, n, transpose_cols);
  else
    hipLaunchKernelGGL(to_f32_kernel<float>, grid, block, 0, s, static_cast<const float*>(src),
                       dst, n, transpose_cols);
  return hipGetLastError();
}

}  // namespace ae
