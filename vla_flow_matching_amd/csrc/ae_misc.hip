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
// against a wide weight that is read once.  A workgroup takes 256 columns:
// thread (column group of 8, K slice) reads its eight columns with one
// 16-byte load per row (bf16), eight rows in flight, over one eighth of
// every 512-row chunk of K; the x values of the chunk sit in LDS.  The eight
// slices' sums are added in slice order through LDS at the end.
constexpr int kGemvThreads = 256;
constexpr int kGvCols = 8;                      // columns per thread
constexpr int kGvGroups = 32;                   // column groups per workgroup
constexpr int kGvSlices = kGemvThreads / kGvGroups;  // K slices per workgroup
constexpr int kGvChunk = 512;                   // rows of K per LDS chunk
constexpr int kGvUnroll = 4;                    // rows in flight per thread

__device__ __forceinline__ float to_f32(bf16_t v) { return bf2f(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ void load8(const T* p, float* w);
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* w) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = __uint_as_float(u[i] << 16);
    w[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* w) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(kGemvThreads) void gemv_rows_kernel(
    const float* X, int ldx, int M, int K, const T* W, int ldw, const T* bias, int N, float* Y,
    int ldy, int act, size_t w_stride, size_t b_stride, size_t y_stride) {
  __shared__ float sx[16][kGvChunk];
  __shared__ float s_red[kGvSlices][kGvGroups * kGvCols];
  const int mat = blockIdx.y;
  W += mat * w_stride;
  bias += mat * b_stride;
  Y += mat * y_stride;
  const int tid = threadIdx.x, grp = tid % kGvGroups, slice = tid / kGvGroups;
  const int n0 = (blockIdx.x * kGvGroups + grp) * kGvCols;
  const bool live = n0 < N;
  const int nc = min(n0, N - kGvCols);  // (a clamped, valid column for idle threads)
  float acc[16][kGvCols];
#pragma unroll
  for (int m = 0; m < 16; ++m)
#pragma unroll
    for (int c = 0; c < kGvCols; ++c) acc[m][c] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kGvChunk) {
    const int kn = min(kGvChunk, K - k0);
    __syncthreads();
    for (int i = tid; i < M * kGvChunk; i += kGemvThreads) {
      const int m = i / kGvChunk, kk = i % kGvChunk;
      sx[m][kk] = kk < kn ? X[static_cast<size_t>(m) * ldx + k0 + kk] : 0.0f;
    }
    __syncthreads();
    // this slice's rows of the chunk: [ks0, ks1)
    const int per = (kn + kGvSlices - 1) / kGvSlices;
    const int ks0 = slice * per, ks1 = min(kn, ks0 + per);
    for (int kk = ks0; kk < ks1; kk += kGvUnroll) {
      // every load of the group issued at a clamped, valid row and masked at
      // use: a guarded load would be waited for on the spot
      float w[kGvUnroll][kGvCols];
#pragma unroll
      for (int u = 0; u < kGvUnroll; ++u)
        load8<T>(W + static_cast<size_t>(k0 + min(kk + u, ks1 - 1)) * ldw + nc, w[u]);
#pragma unroll
      for (int u = 0; u < kGvUnroll; ++u) {
        if (kk + u >= ks1) continue;  // (uniform: the slice's last group)
#pragma unroll
        for (int m = 0; m < 16; ++m)
          if (m < M) {
            const float xv = sx[m][kk + u];
#pragma unroll
            for (int c = 0; c < kGvCols; ++c) acc[m][c] = fmaf(xv, w[u][c], acc[m][c]);
          }
      }
    }
  }
  // the slices' sums, in slice order, one row at a time (plus the bias and
  // the activation), each thread finishing one of the workgroup's columns
  const int n = blockIdx.x * kGvGroups * kGvCols + tid;
  const float bn = n < N ? to_f32(bias[n]) : 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m < M) {  // (uniform)
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kGvCols; ++c) s_red[slice][grp * kGvCols + c] = acc[m][c];
    __syncthreads();
    if (n < N) {
      float y = 0.0f;
#pragma unroll
      for (int sl = 0; sl < kGvSlices; ++sl) y += s_red[sl][tid];
      y += bn;
      if (act == 1) y = silu(y);
      Y[static_cast<size_t>(m) * ldy + n] = y;
    }
    }
  }
  (void)live;
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
                                                          float* rope_cos, float* rope_sin, int extra,
                                                          int* src_of) {
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
    if (vis && src_of) src_of[static_cast<size_t>(b) * P + run] = j;
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

// copy: the visible rows of K and V -> cache keys 0 .. n_valid - 1 in order
// (key-block layout, KvLayout).  grid (L*B*Hkv, max(1, ceil(P/32))), 256
// threads; workgroup y takes keys 32 y .. 32 y + 31, each found through
// src_of (its source row).  K goes row by row, 16 bytes per thread: a key's
// E consecutive dims are contiguous in the cache.  V is transposed in the
// cache (for a dim, E consecutive keys are contiguous), so its rows pass
// through LDS and leave as E keys of one dim per 16-byte store; the keys of
// such a group past n_valid are action-row slots, written with zeros here
// and overwritten by every step's QKV epilogue before attention reads them.
// The first workgroup of each (layer, request, head) also zeroes the keys
// from n_valid + n_act to the end of that 64-key block: attention multiplies
// whole key blocks and relies on the cache being finite there.
constexpr int kCopyRows = 32;

template <typename T>
__global__ __launch_bounds__(256) void prefix_copy_kernel(const T* K, const T* V, const int* src_of,
                                                          const int* n_valid, int n_act, int batch, int P,
                                                          int Hkv, int dh, int Bmax, int S_max,
                                                          T* kcache, T* vtcache) {
  using LY = KvLayout<T>;
  constexpr int E = LY::E;  // elements per 16 bytes
  __shared__ uint4 s_v[kCopyRows * 256 * sizeof(T) / 16];  // V rows of the workgroup's keys (dh <= 256)
  const int lbg = blockIdx.x;
  const int g = lbg % Hkv;
  const int b = (lbg / Hkv) % batch;
  const int l = lbg / (Hkv * batch);
  const int tid = threadIdx.x;
  const int nv = n_valid[b];
  const int key0 = blockIdx.y * kCopyRows;
  const size_t cache_bg = (static_cast<size_t>(l) * Bmax + b) * Hkv + g;
  T* kdst = kcache + cache_bg * S_max * dh;
  T* vdst = vtcache + cache_bg * S_max * dh;
  if (K != nullptr && key0 < nv) {
    const int dq = dh / E;  // 16-byte groups per row
    const size_t row0 = (static_cast<size_t>(l) * batch + b) * P;
    for (int i = tid; i < kCopyRows * dq; i += 256) {
      const int kr = i / dq, q = i % dq, key = key0 + kr;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < nv) {
        const int r = src_of[static_cast<size_t>(b) * P + key];
        const size_t src = ((row0 + r) * Hkv + g) * dh + q * E;
        kv = *reinterpret_cast<const uint4*>(K + src);
        vv = *reinterpret_cast<const uint4*>(V + src);
        *reinterpret_cast<uint4*>(kdst + LY::k_off(key, q * E, dh)) = kv;
      }
      s_v[kr * dq + q] = vv;
    }
    __syncthreads();
    const T* sv = reinterpret_cast<const T*>(s_v);
    for (int i = tid; i < dh * (kCopyRows / E); i += 256) {
      const int d = i % dh, kg = i / dh, k8 = key0 + kg * E;
      if (k8 >= nv) continue;
      T vals[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vals[e] = sv[(kg * E + e) * dh + d];
      *reinterpret_cast<uint4*>(vdst + LY::v_off(k8, d, dh)) = *reinterpret_cast<const uint4*>(vals);
    }
  }
  if (blockIdx.y == 0) {
    // The attention kernels read whole key blocks (at most 64 keys) up to
    // the block holding the request's last key, so only the rest of that
    // block must hold finite values; keys past it are never read.
    const int z0 = min(nv + n_act, S_max);
    const int z1 = min((z0 + 63) / 64 * 64, S_max);
    for (int i = tid; i < (z1 - z0) * dh; i += 256) {
      const int key = z0 + i / dh, d = i % dh;
      kdst[LY::k_off(key, d, dh)] = T(0);
      vdst[LY::v_off(key, d, dh)] = T(0);
    }
  }
}

// The shift term of a norm folded through the next projection:
// out[k][l][n] = sum_d mod[k][l][which][d] W_l[d][n] (adaRMS(h) W =
// r (h (1 + scale)) W + shift W), read straight from the packed fragments, so
// n is in packed column order.  One wave per (16-column block, layer), four
// per workgroup: lane (g, j) holds k-slot g of column j; fp32 sums over d in
// increasing order per step.  The workgroup first copies the modulation rows
// of up to kSbSteps steps into LDS (all loads in flight), then streams its
// weight fragments eight at a time and adds every step's products from LDS,
// so each fragment is read once per pass instead of once per step.
constexpr int kSbSteps = 16;     // steps per pass at most
constexpr int kSbWaves = 4;      // column blocks per workgroup
constexpr int kSbFill = 16;      // float4 per thread per round of the LDS fill
constexpr int kSbLdsFloats = 16384;  // 64 KiB of modulation rows per pass at most

__host__ __device__ inline int shift_bias_steps_per_pass(int K, int n_steps) {
  int sp = kSbLdsFloats / K;
  if (sp > kSbSteps) sp = kSbSteps;
  if (sp > n_steps) sp = n_steps;
  return sp < 1 ? 1 : sp;
}

template <typename T>
__global__ __launch_bounds__(kSbWaves * kWave) void shift_bias_kernel(const uint4* W, size_t layer_stride, int K,
                                                                      int N, const float* mod, int n_steps, int L,
                                                                      int D, int nchunk, int which, float* out) {
  constexpr int E = Mma<T>::E, KSTEP = Mma<T>::KSTEP;
  extern __shared__ float s_sh[];  // [steps of the pass][K]
  const int l = blockIdx.y, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane / 16;
  const int nbs = N / 16;
  const int nb = blockIdx.x * kSbWaves + wave;  // this wave's column block (past the last: idle)
  const int k_frags = K / KSTEP;
  const int sp = shift_bias_steps_per_pass(K, n_steps);
  const uint4* Wf = W + l * layer_stride + static_cast<size_t>(min(nb, nbs - 1)) * k_frags * kWave + lane;
  for (int k0 = 0; k0 < n_steps; k0 += sp) {
    const int ns = min(sp, n_steps - k0);
    __syncthreads();  // (the previous pass is done with the rows)
    const int n4 = ns * (K / 4);
    for (int i0 = 0; i0 < n4; i0 += kSbFill * kSbWaves * kWave) {
      float4 v[kSbFill];
#pragma unroll
      for (int u = 0; u < kSbFill; ++u) {
        const int i = min(i0 + u * kSbWaves * kWave + tid, n4 - 1);
        const int kk = (4 * i) / K, d = (4 * i) % K;
        v[u] = *reinterpret_cast<const float4*>(mod + ((static_cast<size_t>(k0 + kk) * L + l) * nchunk + which) * D + d);
      }
#pragma unroll
      for (int u = 0; u < kSbFill; ++u) {
        const int i = i0 + u * kSbWaves * kWave + tid;
        if (i < n4) reinterpret_cast<float4*>(s_sh)[i] = v[u];
      }
    }
    __syncthreads();
    float acc[kSbSteps];
#pragma unroll
    for (int kk = 0; kk < kSbSteps; ++kk) acc[kk] = 0.0f;
    for (int kf0 = 0; kf0 < k_frags; kf0 += 8) {
      uint4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = Wf[static_cast<size_t>(min(kf0 + u, k_frags - 1)) * kWave];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (kf0 + u >= k_frags) break;
        const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
        float wv[E];
#pragma unroll
        for (int i = 0; i < E; ++i)
          wv[i] = sizeof(T) == 2 ? __uint_as_float((wd[i / 2] >> (16 * (i % 2))) << 16) : __uint_as_float(wd[i % 4]);
        const int d0 = (kf0 + u) * KSTEP + E * g;
#pragma unroll
        for (int kk = 0; kk < kSbSteps; ++kk) {
          if (kk >= ns) break;
          const float* sh = s_sh + kk * K + d0;
#pragma unroll
          for (int i = 0; i < E; ++i) acc[kk] += sh[i] * wv[i];
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < kSbSteps; ++kk) {
      if (kk >= ns) break;
      float a = acc[kk];
      a += __shfl_xor(a, 16, kWave);
      a += __shfl_xor(a, 32, kWave);
      if (lane < 16 && nb < nbs) out[(static_cast<size_t>(k0 + kk) * L + l) * N + 16 * nb + lane] = a;
    }
  }
}

}  // namespace

hipError_t launch_shift_bias(Dt dt, const uint4* W, size_t layer_stride, int K, int N, const float* mod,
                             int n_steps, int L, int D, int nchunk, int which, float* out, hipStream_t s) {
  if (N % 16 || K % 32 || K > D || n_steps < 1 || L < 1 || which < 0 || which >= nchunk)
    return hipErrorInvalidValue;
  dim3 grid((N / 16 + kSbWaves - 1) / kSbWaves, L), block(kSbWaves * kWave);
  const size_t lds = static_cast<size_t>(shift_bias_steps_per_pass(K, n_steps)) * K * sizeof(float);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(shift_bias_kernel<bf16_t>, grid, block, lds, s, W, layer_stride, K, N, mod, n_steps, L,
                       D, nchunk, which, out);
  else
    hipLaunchKernelGGL(shift_bias_kernel<float>, grid, block, lds, s, W, layer_stride, K, N, mod, n_steps, L, D,
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
  if (M < 1 || M > 16 || N < kGvCols || N % kGvCols || ldw % kGvCols) return hipErrorInvalidValue;
  const int cols_per_block = kGvGroups * kGvCols;
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
                              hipStream_t s, int extra, int* src_of) {
  hipLaunchKernelGGL(prefix_scan_kernel, dim3(batch), dim3(256), 0, s, mask, P, comp_idx, n_valid,
                     T, dh, theta, rope_cos, rope_sin, extra, src_of);
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

hipError_t launch_prefix_copy(Dt dt, const void* K, const void* V, const int* src_of,
                              const int* n_valid, int n_act, int L, int batch, int P, int Hkv, int dh,
                              int Bmax, int S_max, void* kcache, void* vtcache, hipStream_t s) {
  if (dh > 256) return hipErrorInvalidValue;
  dim3 grid(L * batch * Hkv, P > 0 ? (P + kCopyRows - 1) / kCopyRows : 1), block(256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(prefix_copy_kernel<bf16_t>, grid, block, 0, s,
                       static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V), src_of, n_valid,
                       n_act, batch, P, Hkv, dh, Bmax, S_max, static_cast<bf16_t*>(kcache),
                       static_cast<bf16_t*>(vtcache));
  else
    hipLaunchKernelGGL(prefix_copy_kernel<float>, grid, block, 0, s, static_cast<const float*>(K),
                       static_cast<const float*>(V), src_of, n_valid, n_act, batch, P, Hkv, dh, Bmax,
                       S_max, static_cast<float*>(kcache), static_cast<float*>(vtcache));
  return hipGetLastError();
}

}  // namespace ae
