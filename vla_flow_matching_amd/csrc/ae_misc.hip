// The small kernels around the layer stack: the time path (once per call),
// the action-in and final-norm / action-out / Euler kernels (once per step),
// and prefix ingest (once per query).
#include <math.h>

#include <algorithm>

#include "ae_device.h"
#include "ae_kernels.h"

namespace ae {

namespace {

// ---------------------------------------------------------------------------
// Time path.  Step k evaluates the velocity at t_k = (N - k)/N; its
// sinusoidal embedding is [sin(2 pi t / P_i) | cos(2 pi t / P_i)], i < D/2,
// with periods P_i geometric from 4e-3 to 4.0.  Computed in double: the
// angles reach ~1.6e3 rad at t = 1.  The whole path depends only on t, so
// it runs once per call (sglang PR summary, implementation item 2).
// ---------------------------------------------------------------------------

__global__ void tpath_sinusoid_kernel(float* e, int n_steps, int width) {
  const int k = blockIdx.x;
  const int half = width / 2;
  const double t = static_cast<double>(n_steps - k) / static_cast<double>(n_steps);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double frac = static_cast<double>(i) / static_cast<double>(half - 1);
    const double period = 4e-3 * pow(1000.0, frac);
    const double ang = 2.0 * M_PI * t / period;
    e[static_cast<size_t>(k) * width + i] = static_cast<float>(sin(ang));
    e[static_cast<size_t>(k) * width + half + i] = static_cast<float>(cos(ang));
  }
}

// Y[m][n] = act(sum_k X[m][k] W[k][n] + b[n]) for m < M <= 16: a few rows
// against a wide weight that is read once.  Two columns per thread, 512 per
// block; the k loop keeps 16 independent weight loads in flight per thread.
constexpr int kGemvThreads = 256;
constexpr int kGemvCols = 2;
constexpr int kGemvK = 256;
constexpr int kGemvUnroll = 16;

template <typename T> __device__ __forceinline__ void load2(const T* p, float* w);
template <> __device__ __forceinline__ void load2<bf16_t>(const bf16_t* p, float* w) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  w[0] = __uint_as_float(v << 16);
  w[1] = __uint_as_float(v & 0xffff0000u);
}
template <> __device__ __forceinline__ void load2<float>(const float* p, float* w) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  w[0] = v.x;
  w[1] = v.y;
}

template <typename T>
__global__ __launch_bounds__(kGemvThreads) void gemv_rows_kernel(
    const float* X, int ldx, int M, int K, const T* W, int ldw, const T* bias, int N, float* Y,
    int ldy, int act, size_t w_stride, size_t b_stride, size_t y_stride) {
  __shared__ float sx[16][kGemvK];
  const int mat = blockIdx.y;
  W += mat * w_stride;
  bias += mat * b_stride;
  Y += mat * y_stride;
  const int n0 = (blockIdx.x * kGemvThreads + threadIdx.x) * kGemvCols;
  const bool live = n0 < N;
  float acc[16][kGemvCols];
#pragma unroll
  for (int m = 0; m < 16; ++m)
#pragma unroll
    for (int c = 0; c < kGemvCols; ++c) acc[m][c] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kGemvK) {
    const int kn = min(kGemvK, K - k0);
    __syncthreads();
    for (int i = threadIdx.x; i < M * kGemvK; i += kGemvThreads) {
      const int m = i / kGemvK, kk = i % kGemvK;
      sx[m][kk] = kk < kn ? X[static_cast<size_t>(m) * ldx + k0 + kk] : 0.0f;
    }
    __syncthreads();
    if (!live) continue;
    for (int kk = 0; kk < kn; kk += kGemvUnroll) {
      // every load of the group issued at a clamped, valid row and masked
      // at use: a guarded load would be waited for on the spot, one HBM
      // round trip per row
      float w[kGemvUnroll][kGemvCols];
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u)
        load2<T>(W + static_cast<size_t>(k0 + min(kk + u, kn - 1)) * ldw + n0, w[u]);
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u)
        if (kk + u >= kn) w[u][0] = w[u][1] = 0.0f;
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u)
#pragma unroll
        for (int m = 0; m < 16; ++m)
          if (m < M) {
            const float xv = sx[m][kk + u];
#pragma unroll
            for (int c = 0; c < kGemvCols; ++c) acc[m][c] = fmaf(xv, w[u][c], acc[m][c]);
          }
    }
  }
  if (!live) return;
  float bv[kGemvCols];
  load2<T>(bias + n0, bv);
#pragma unroll
  for (int m = 0; m < 16; ++m)
    if (m < M)
#pragma unroll
      for (int c = 0; c < kGemvCols; ++c) {
        float y = acc[m][c] + bv[c];
        if (act == 1) y = silu(y);
        Y[static_cast<size_t>(m) * ldy + n0 + c] = y;
      }
}

// ---------------------------------------------------------------------------
// Action-in projection h = x W_in + b_in, plus per-64-column partial row sums
// of h^2 for the first layer's adaRMS.  grid (ceil(M/8), ceil(D/256)), 256
// threads: thread t owns column n of eight rows, loads its W_in column once
// (all of it in flight) and reuses it for the rows; the rows' x values are
// staged in LDS once per workgroup.
// ---------------------------------------------------------------------------
constexpr int kInRows = 8;

template <int AMAX>
__global__ __launch_bounds__(256) void action_in_kernel(const float* x, int M, int A, const float* w_in,
                                                        const float* b_in, float* h, int D,
                                                        float* ssq, int ldssq, uint16_t* ha,
                                                        const float* sc) {
  __shared__ float s_x[kInRows][AMAX];
  const int m0 = blockIdx.x * kInRows;
  const int n = blockIdx.y * 256 + threadIdx.x;
  // the workgroup's x rows once, into LDS (rows past M and columns past A
  // read clamped entries and are never used)
  for (int i = threadIdx.x; i < kInRows * AMAX; i += 256)
    s_x[i / AMAX][i % AMAX] = x[min(m0 + i / AMAX, M - 1) * A + min(i % AMAX, A - 1)];
  __syncthreads();
  if (n >= D) return;  // (D % 64 == 0: whole waves; no barriers below)
  // every load unconditional and in bounds (indices clamped, masked at use),
  // so all of them are in flight together
  float w[AMAX];
#pragma unroll
  for (int a = 0; a < AMAX; ++a) w[a] = w_in[static_cast<size_t>(min(a, A - 1)) * D + n];
  const float bn = b_in[n];
  const float hs = ha ? 1.0f + sc[n] : 0.0f;
  for (int r = 0; r < kInRows; ++r) {
    const int m = m0 + r;
    if (m >= M) break;
    float acc = 0.0f;
#pragma unroll
    for (int a = 0; a < AMAX; ++a) acc = fmaf(s_x[r][a], a < A ? w[a] : 0.0f, acc);
    acc += bn;
    h[static_cast<size_t>(m) * D + n] = acc;
    if (ha) ha[static_cast<size_t>(m) * D + n] = f2bf(acc * hs);
    const float sq = wave_sum(acc * acc);
    if (threadIdx.x % kWave == 0) ssq[static_cast<size_t>(n / 64) * ldssq + m] = sq;
  }
}

// ---------------------------------------------------------------------------
// Final adaRMS, action-out projection and the Euler update of one row:
// v = adaRMS(h; scale_f, shift_f) W_out + b_out, x += dt v.  grid M, 256
// threads: thread t holds the row's columns t + 256 j (j < KJ) in registers
// and forms partial dot products for 32 outputs at a time with all of its
// W_out loads in flight (W_out held transposed, [A][D]: consecutive threads
// read consecutive columns); each output is then summed over the workgroup.
// ---------------------------------------------------------------------------

constexpr int kMaxWidth = 4096;
constexpr int kOutChunk = 32;  // outputs per pass

template <int KJ>
__global__ __launch_bounds__(256) void action_out_kernel(float* x, int A, const float* h, int D,
                                                         const float* scale, const float* shift,
                                                         float eps, const float* w_out_t,
                                                         const float* b_out, float dt) {
  __shared__ float s_red[4][kOutChunk];
  __shared__ float s_ss[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const float* hr = h + static_cast<size_t>(m) * D;
  // columns past D: clamped loads, zero values
  float u[KJ];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int k = tid + 256 * j;
    u[j] = k < D ? hr[min(k, D - 1)] : 0.0f;
    ss = fmaf(u[j], u[j], ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) s_ss[wave] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((s_ss[0] + s_ss[1] + s_ss[2] + s_ss[3]) / static_cast<float>(D) + eps);
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int k = min(tid + 256 * j, D - 1);
    const float v = u[j] * r * (1.0f + scale[k]) + shift[k];
    u[j] = tid + 256 * j < D ? v : 0.0f;
  }
  for (int a0 = 0; a0 < A; a0 += kOutChunk) {
    float acc[kOutChunk];
#pragma unroll
    for (int i = 0; i < kOutChunk; ++i) {
      // outputs past A read row A - 1 and are never stored
      const float* wr = w_out_t + static_cast<size_t>(min(a0 + i, A - 1)) * D;
      acc[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < KJ; ++j) acc[i] = fmaf(u[j], wr[min(tid + 256 * j, D - 1)], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < kOutChunk; ++i) {
      const float t = wave_sum(acc[i]);
      if (lane == 0) s_red[wave][i] = t;
    }
    __syncthreads();
    if (tid < kOutChunk && a0 + tid < A) {
      const int a = a0 + tid;
      const float v = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
      x[m * A + a] += dt * (v + b_out[a]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Prefix ingest.
// scan: per request, the visible count n_b and each visible row's compacted
// index (prefix order kept); then the RoPE tables of the action tokens at
// positions n_b + t (pads do not advance positions: LoongForge blog,
// section 1), computed in double.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void prefix_scan_kernel(const uint8_t* mask, int P, int* comp_idx,
                                                          int* n_valid, int T, int dh, float theta,
                                                          float* rope_cos, float* rope_sin, int extra) {
  __shared__ int s_cnt[256];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int chunk = (P + 255) / 256;
  const int j0 = min(P, tid * chunk), j1 = min(P, j0 + chunk);
  int c = 0;
  for (int j = j0; j < j1; ++j) c += mask[static_cast<size_t>(b) * P + j] != 0;
  s_cnt[tid] = c;
  __syncthreads();
  // inclusive scan (Hillis-Steele)
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? s_cnt[tid - off] : 0;
    __syncthreads();
    s_cnt[tid] += v;
    __syncthreads();
  }
  int run = s_cnt[tid] - c;
  for (int j = j0; j < j1; ++j) {
    const bool vis = mask[static_cast<size_t>(b) * P + j] != 0;
    comp_idx[static_cast<size_t>(b) * P + j] = vis ? run : -1;
    run += vis;
  }
  const int nv = s_cnt[255] + extra;
  if (tid == 0) n_valid[b] = nv;
  const int half = dh / 2;
  for (int i = tid; i < T * half; i += 256) {
    const int t = i / half, j = i % half;
    const double w = pow(static_cast<double>(theta), -2.0 * j / dh);
    const double ph = static_cast<double>(nv + t) * w;
    rope_cos[(static_cast<size_t>(b) * T + t) * half + j] = static_cast<float>(cos(ph));
    rope_sin[(static_cast<size_t>(b) * T + t) * half + j] = static_cast<float>(sin(ph));
  }
}

// copy: visible row j of K and V -> cache key comp_idx[j] (key-block layout,
// KvLayout).  grid (L*B*Hkv, max(1, ceil(P/32))), 256 threads.  The first
// row block of each (layer, request, head) also zeroes the keys from the
// request's n_valid + n_act to the end of that 64-key block: attention
// multiplies whole key blocks and relies on the cache being finite there.
constexpr int kCopyRows = 32;

template <typename T>
__global__ __launch_bounds__(256) void prefix_copy_kernel(const T* K, const T* V, const int* comp_idx,
                                                          const int* n_valid, int n_act, int batch, int P,
                                                          int Hkv, int dh, int Bmax, int S_max,
                                                          T* kcache, T* vtcache) {
  using LY = KvLayout<T>;
  __shared__ int sci[kCopyRows];
  const int lbg = blockIdx.x;
  const int g = lbg % Hkv;
  const int b = (lbg / Hkv) % batch;
  const int l = lbg / (Hkv * batch);
  const int j0 = blockIdx.y * kCopyRows;
  const int nrows = min(kCopyRows, P - j0);
  if (threadIdx.x < kCopyRows)
    sci[threadIdx.x] = threadIdx.x < nrows ? comp_idx[static_cast<size_t>(b) * P + j0 + threadIdx.x] : -1;
  __syncthreads();
  const size_t src_row0 = ((static_cast<size_t>(l) * batch + b) * P + j0) * Hkv + g;
  const size_t cache_bg = (static_cast<size_t>(l) * Bmax + b) * Hkv + g;
  T* kdst = kcache + cache_bg * S_max * dh;
  T* vdst = vtcache + cache_bg * S_max * dh;
  for (int i = threadIdx.x; i < nrows * dh; i += 256) {
    const int r = i / dh, d = i % dh;
    const int ci = sci[r];
    if (ci < 0) continue;  // invisible row: never read
    const size_t src = (src_row0 + static_cast<size_t>(r) * Hkv) * dh + d;
    kdst[LY::k_off(ci, d, dh)] = K[src];
    vdst[LY::v_off(ci, d, dh)] = V[src];
  }
  if (blockIdx.y == 0) {
    // The attention kernels read whole key blocks (at most 64 keys) up to
    // the block holding the request's last key, so only the rest of that
    // block must hold finite values; keys past it are never read.
    const int z0 = min(n_valid[b] + n_act, S_max);
    const int z1 = min((z0 + 63) / 64 * 64, S_max);
    for (int i = threadIdx.x; i < (z1 - z0) * dh; i += 256) {
      const int key = z0 + i / dh, d = i % dh;
      kdst[LY::k_off(key, d, dh)] = T(0);
      vdst[LY::v_off(key, d, dh)] = T(0);
    }
  }
}

// The shift term of a norm folded through the next projection:
// out[k][l][n] = sum_d mod[k][l][which][d] W_l[d][n] (adaRMS(h) W =
// r (h (1 + scale)) W + shift W), read straight from the packed fragments, so
// n is in packed column order.  One wave per (16-column block, layer): lane
// (g, j) holds k-slot g of column j; fp32 sums, one step at a time.
template <typename T>
__global__ void shift_bias_kernel(const uint4* W, size_t layer_stride, int K, int N, const float* mod,
                                  int n_steps, int L, int D, int nchunk, int which, float* out) {
  constexpr int E = Mma<T>::E, KSTEP = Mma<T>::KSTEP;
  const int nb = blockIdx.x, l = blockIdx.y, lane = threadIdx.x, g = lane / 16;
  const int k_frags = K / KSTEP;
  const uint4* Wf = W + l * layer_stride + static_cast<size_t>(nb) * k_frags * kWave + lane;
  for (int k = 0; k < n_steps; ++k) {
    const float* sh = mod + ((static_cast<size_t>(k) * L + l) * nchunk + which) * D;
    float acc = 0.0f;
    for (int kf = 0; kf < k_frags; ++kf) {
      const uint4 w = Wf[static_cast<size_t>(kf) * kWave];
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      const int d0 = kf * KSTEP + E * g;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float wv = sizeof(T) == 2 ? __uint_as_float((wd[i / 2] >> (16 * (i % 2))) << 16)
                                        : __uint_as_float(wd[i % 4]);
        acc += sh[d0 + i] * wv;
      }
    }
    acc += __shfl_xor(acc, 16, kWave);
    acc += __shfl_xor(acc, 32, kWave);
    if (lane < 16) out[(static_cast<size_t>(k) * L + l) * N + 16 * nb + lane] = acc;
  }
}

}  // namespace

hipError_t launch_shift_bias(Dt dt, const uint4* W, size_t layer_stride, int K, int N, const float* mod,
                             int n_steps, int L, int D, int nchunk, int which, float* out, hipStream_t s) {
  if (N % 16 || K % 32 || K > D || n_steps < 1 || L < 1 || which < 0 || which >= nchunk)
    return hipErrorInvalidValue;
  dim3 grid(N / 16, L), block(kWave);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(shift_bias_kernel<bf16_t>, grid, block, 0, s, W, layer_stride, K, N, mod, n_steps, L,
                       D, nchunk, which, out);
  else
    hipLaunchKernelGGL(shift_bias_kernel<float>, grid, block, 0, s, W, layer_stride, K, N, mod, n_steps, L, D,
                       nchunk, which, out);
  return hipGetLastError();
}

namespace {
__global__ void zero_ints_kernel(int* p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}
}  // namespace

hipError_t launch_zero_ints(int* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = static_cast<int>(std::min<size_t>(64, (n + 255) / 256));
  hipLaunchKernelGGL(zero_ints_kernel, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_tpath_sinusoid(float* e, int n_steps, int width, hipStream_t s) {
  hipLaunchKernelGGL(tpath_sinusoid_kernel, dim3(n_steps), dim3(256), 0, s, e, n_steps, width);
  return hipGetLastError();
}

hipError_t launch_gemv_rows(Dt dt, const float* X, int ldx, int M, int K, const void* W, int ldw,
                            const void* b, int N, float* Y, int ldy, int act, int n_mat,
                            size_t w_stride, size_t b_stride, size_t y_stride, hipStream_t s) {
  if (M < 1 || M > 16 || N % kGemvCols || ldw % kGemvCols) return hipErrorInvalidValue;
  const int cols_per_block = kGemvThreads * kGemvCols;
  dim3 grid((N + cols_per_block - 1) / cols_per_block, n_mat), block(kGemvThreads);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(gemv_rows_kernel<bf16_t>, grid, block, 0, s, X, ldx, M, K,
                       static_cast<const bf16_t*>(W), ldw, static_cast<const bf16_t*>(b), N, Y,
                       ldy, act, w_stride, b_stride, y_stride);
  else
    hipLaunchKernelGGL(gemv_rows_kernel<float>, grid, block, 0, s, X, ldx, M, K,
                       static_cast<const float*>(W), ldw, static_cast<const float*>(b), N, Y, ldy,
                       act, w_stride, b_stride, y_stride);
  return hipGetLastError();
}

hipError_t launch_action_in(const float* x, int M, int A, const float* w_in, const float* b_in,
                            float* h, int D, float* ssq, int ldssq, hipStream_t s, uint16_t* ha,
                            const float* sc) {
  if ((ha == nullptr) != (sc == nullptr) || D % 64 || A < 1 || A > 64) return hipErrorInvalidValue;
  const dim3 grid((M + kInRows - 1) / kInRows, (D + 255) / 256);
  if (A <= 32)
    hipLaunchKernelGGL(action_in_kernel<32>, grid, dim3(256), 0, s, x, M, A, w_in, b_in, h, D, ssq, ldssq, ha, sc);
  else
    hipLaunchKernelGGL(action_in_kernel<64>, grid, dim3(256), 0, s, x, M, A, w_in, b_in, h, D, ssq, ldssq, ha, sc);
  return hipGetLastError();
}

hipError_t launch_action_out(float* x, int M, int A, const float* h, int D, const float* scale,
                             const float* shift, float eps, const float* w_out,
                             const float* b_out, float dt, hipStream_t s) {
  if (D > kMaxWidth || A < 1) return hipErrorInvalidValue;
  const int kj = (D + 255) / 256;
#define AE_OUT(KJV)                                                                                   \
  if (kj <= KJV) {                                                                                    \
    hipLaunchKernelGGL(action_out_kernel<KJV>, dim3(M), dim3(256), 0, s, x, A, h, D, scale, shift, eps, \
                       w_out, b_out, dt);                                                             \
    return hipGetLastError();                                                                         \
  }
  AE_OUT(1)
  AE_OUT(2)
  AE_OUT(3)
  AE_OUT(4)
  AE_OUT(8)
  AE_OUT(16)
#undef AE_OUT
  return hipErrorInvalidValue;
}

hipError_t launch_prefix_scan(const uint8_t* mask, int batch, int P, int* comp_idx, int* n_valid,
                              int T, int dh, float theta, float* rope_cos, float* rope_sin,
                              hipStream_t s, int extra) {
  hipLaunchKernelGGL(prefix_scan_kernel, dim3(batch), dim3(256), 0, s, mask, P, comp_idx, n_valid,
                     T, dh, theta, rope_cos, rope_sin, extra);
  return hipGetLastError();
}

namespace {

// cos / sin of RoPE at positions 0 .. n_pos - 1 (double math, fp32 table):
// the count positions of context rows
__global__ void pos_table_kernel(int n_pos, int dh, float theta, float* cos_t, float* sin_t) {
  const int half = dh / 2;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_pos * half; i += gridDim.x * blockDim.x) {
    const int pos = i / half, j = i % half;
    const double w = pow(static_cast<double>(theta), -2.0 * j / dh);
    const double ph = static_cast<double>(pos) * w;
    cos_t[i] = static_cast<float>(cos(ph));
    sin_t[i] = static_cast<float>(sin(ph));
  }
}

// The robot state's context row (256 columns of request blockIdx.y per
// workgroup): fp32 sums of the state times the input layer in state order,
// plus its bias, stored as bf16; its cache key is the request's last visible
// position.  The state's weights are requested 8 rows at a time, all in
// flight (a loop bounded at run time would wait out each load in turn).
constexpr int kStateBatch = 8;
__global__ __launch_bounds__(256) void state_prep_kernel(const float* state, int S, const bf16_t* w,
                                                         const bf16_t* bias, int D, const int* n_valid,
                                                         bf16_t* out, int* key_out) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < D) {
    float acc = bf2f(bias[c]);
    for (int i0 = 0; i0 < S; i0 += kStateBatch) {
      float sv[kStateBatch], wv[kStateBatch];
#pragma unroll
      for (int u = 0; u < kStateBatch; ++u) {
        const int i = min(i0 + u, S - 1);
        sv[u] = state[static_cast<size_t>(b) * S + i];
        wv[u] = bf2f(w[static_cast<size_t>(i) * D + c]);
      }
#pragma unroll
      for (int u = 0; u < kStateBatch; ++u)
        if (i0 + u < S) acc = fmaf(sv[u], wv[u], acc);
    }
    out[static_cast<size_t>(b) * D + c] = f2bf(acc);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) key_out[b] = n_valid[b] - 1;
}

}  // namespace

hipError_t launch_pos_table(int n_pos, int dh, float theta, float* cos_t, float* sin_t, hipStream_t s) {
  if (n_pos < 1 || dh < 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pos_table_kernel, dim3(256), dim3(256), 0, s, n_pos, dh, theta, cos_t, sin_t);
  return hipGetLastError();
}

hipError_t launch_state_prep(const float* state, int batch, int S, const uint16_t* w, const uint16_t* bias,
                             int D, const int* n_valid, uint16_t* out, int* key_out, hipStream_t s) {
  if (batch < 1 || S < 1 || D < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(state_prep_kernel, dim3((D + 255) / 256, batch), dim3(256), 0, s, state, S, w, bias, D,
                     n_valid, out, key_out);
  return hipGetLastError();
}

hipError_t launch_prefix_copy(Dt dt, const void* K, const void* V, const int* comp_idx,
                              const int* n_valid, int n_act, int L, int batch, int P, int Hkv, int dh,
                              int Bmax, int S_max, void* kcache, void* vtcache, hipStream_t s) {
  if (dh > 256) return hipErrorInvalidValue;
  dim3 grid(L * batch * Hkv, P > 0 ? (P + kCopyRows - 1) / kCopyRows : 1), block(256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(prefix_copy_kernel<bf16_t>, grid, block, 0, s,
                       static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V), comp_idx, n_valid,
                       n_act, batch, P, Hkv, dh, Bmax, S_max, static_cast<bf16_t*>(kcache),
                       static_cast<bf16_t*>(vtcache));
  else
    hipLaunchKernelGGL(prefix_copy_kernel<float>, grid, block, 0, s, static_cast<const float*>(K),
                       static_cast<const float*>(V), comp_idx, n_valid, n_act, batch, P, Hkv, dh, Bmax,
                       S_max, static_cast<float*>(kcache), static_cast<float*>(vtcache));
  return hipGetLastError();
}

}  // namespace ae
