// Test-only entry points (include/ae_testing.h): single pieces of the fp8
// e4m3 projection path run on inputs a test chooses, through the same
// kernels the batched denoise path launches (quant_kernel, rownorm_kernel,
// the weight amax / scale / packing kernels and tgemm_kernel with its QKV,
// gelu and residual epilogues).  The small kernels here only adapt inputs
// and outputs (a row-block amax, a fill, read-back of the key-block cache).
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "../../include/ae_testing.h"
#include "ae_device.h"
#include "ae_kernels.h"

using namespace ae;

namespace {

constexpr int kTargetBlocks = 256;

// rowmax[blk][row] = max |x[row][64 blk .. 64 blk + 63]|; grid (K / 64, M), 64 threads
__global__ void rowblock_amax_kernel(const float* x, int M, int K, float* rowmax) {
  const int blk = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
  float v = fabsf(x[static_cast<size_t>(row) * K + 64 * blk + lane]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  if (lane == 0) rowmax[static_cast<size_t>(blk) * M + row] = v;
}

__global__ void fill_kernel(float* p, size_t n, float v) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

__global__ void bf16_to_f32_kernel(const bf16_t* src, size_t n, float* dst) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = bf2f(src[i]);
}

// out[row][hd dh + d] = cache entry of key `row`, dim d of head hd (one
// request; key-block layout); is_v selects the V layout.
__global__ void unpack_cache_kernel(const bf16_t* cache, int M, int Hkv, int dh, int S_max, int is_v,
                                    float* out) {
  using LY = KvLayout<bf16_t>;
  const size_t n = static_cast<size_t>(M) * Hkv * dh;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int row = static_cast<int>(i / (static_cast<size_t>(Hkv) * dh));
    const int hd = static_cast<int>((i / dh) % Hkv), d = static_cast<int>(i % dh);
    const size_t off = static_cast<size_t>(hd) * S_max * dh + (is_v ? LY::v_off(row, d, dh) : LY::k_off(row, d, dh));
    out[i] = bf2f(cache[off]);
  }
}

// Device scratch of one call, freed when the call returns.
struct Scratch {
  std::vector<void*> ptrs;
  hipError_t err = hipSuccess;
  template <typename P>
  P* get(size_t bytes) {
    void* p = nullptr;
    if (err == hipSuccess) err = hipMalloc(&p, bytes ? bytes : 16);
    if (err != hipSuccess) return nullptr;
    ptrs.push_back(p);
    return static_cast<P*>(p);
  }
  ~Scratch() {
    for (void* p : ptrs) (void)hipFree(p);
  }
};

// Wait for the stream (also after a failed launch: the scratch is freed
// next, and work queued before the failure may still read it).
ae_status finish(hipError_t e, hipStream_t s) {
  const hipError_t w = hipStreamSynchronize(s);
  if (e == hipSuccess) e = w;
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return AE_ERR_HIP;
  }
  return AE_OK;
}

#define AE_T(call)                            \
  do {                                        \
    hipError_t e_ = (call);                   \
    if (e_ != hipSuccess) return finish(e_, s); \
  } while (0)

// Per-tensor amax of bf16 weights -> (448 / amax, amax / 448) in mul[i], sc[i].
hipError_t weight_scales(const uint16_t* const* w, const size_t* n, int count, unsigned* amax, float* mul,
                         float* sc, hipStream_t s) {
  hipError_t e = hipMemsetAsync(amax, 0, sizeof(unsigned) * count, s);
  for (int i = 0; e == hipSuccess && i < count; ++i) e = launch_weight_amax(w[i], n[i], amax + i, s);
  if (e == hipSuccess) e = launch_fp8_scales(amax, count, mul, sc, s);
  return e;
}

TGemmArgs gemm_args(const TGemmPlan& g, const uint8_t* codes, const float* sx_row, int M, int N, int K,
                    const uint4* W, float* partial, const float* sw) {
  TGemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = codes;
  a.lda_bytes = static_cast<size_t>(K);
  a.M = M; a.N = N; a.K = K;
  a.W = W;
  a.n_tiles = g.n_tiles; a.m_tiles = g.m_tiles; a.ksplit = g.ksplit; a.bm = g.bm;
  a.partial = partial;
  a.sx_row = sx_row;
  a.sw = sw;
  return a;
}

}  // namespace

extern "C" {

ae_status aetest_fp8_quantize(const float* x, int M, int K, int T, uint8_t* codes, float* sx_row,
                              void* stream) {
  if (!x || !codes || !sx_row || M < 1 || T < 1 || M % T || K < 64 || K % 64) return AE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch sc;
  float* rowmax = sc.get<float>(static_cast<size_t>(K / 64) * M * 4);
  AE_T(sc.err);
  hipLaunchKernelGGL(rowblock_amax_kernel, dim3(K / 64, M), dim3(kWave), 0, s, x, M, K, rowmax);
  AE_T(hipGetLastError());
  AE_T(launch_quant(x, nullptr, nullptr, nullptr, nullptr, M, K, T, rowmax, K / 64, M, codes, sx_row, s));
  return finish(hipSuccess, s);
}

ae_status aetest_fp8_norm_quantize(const float* h, int M, int D, int T, const float* scale, const float* shift,
                                   float eps, uint8_t* codes, float* sx_row, float* r_out, void* stream) {
  if (!h || !scale || !shift || !codes || !sx_row || !r_out || M < 1 || T < 1 || M % T || D < 64 || D % 64 ||
      D > 4096 || !(eps >= 0.0f))
    return AE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch sc;
  float* rowmax = sc.get<float>(static_cast<size_t>(M) * 4);
  AE_T(sc.err);
  if (T == 1) {  // a scale per row: the one-pass row-wise kernel
    AE_T(launch_rownorm_quant(h, M, D, scale, shift, eps, r_out, codes, sx_row, s));
    return finish(hipSuccess, s);
  }
  AE_T(launch_rownorm(h, M, D, scale, shift, eps, r_out, rowmax, s));
  AE_T(launch_quant(nullptr, h, r_out, scale, shift, M, D, T, rowmax, 1, M, codes, sx_row, s));
  return finish(hipSuccess, s);
}

ae_status aetest_fp8_down(const uint8_t* codes, const float* sx_row, int M, int K, const uint16_t* w, int N,
                          float* y, float* sw, int per_column, void* stream) {
  if (!codes || !sx_row || !w || !y || !sw || M < 1) return AE_ERR_INVALID_ARGUMENT;
  if (K < 128 || K % 128 || N < 128 || N % 128) return AE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const TGemmPlan g = plan_tgemm(M, N, K, tgemm_kc(OP_FP8), kTargetBlocks);
  Scratch sc;
  uint4* packed = sc.get<uint4>(static_cast<size_t>(K) * N);
  unsigned* amax = sc.get<unsigned>(4);
  float* mul = sc.get<float>(4);
  float* gate = sc.get<float>(static_cast<size_t>(N) * 4);
  float* partial = sc.get<float>(tgemm_partial_floats(g) * 4);
  float* cmul = sc.get<float>(static_cast<size_t>(N) * 4);
  float* swc = sc.get<float>(static_cast<size_t>(N) * 4);
  AE_T(sc.err);
  if (per_column) {
    AE_T(launch_fp8_col_scales(w, K, N, N, cmul, sw, s));
    AE_T(launch_pack_fp8(PACK_PLAIN, w, nullptr, nullptr, K, N, N, 0, 0, 1, 1, 64, cmul, packed, s, cmul));
    AE_T(launch_pack_col_scales(PACK_PLAIN, sw, nullptr, nullptr, N, 1, 1, 64, swc, s));
  } else {
    const uint16_t* ws[1] = {w};
    const size_t ns[1] = {static_cast<size_t>(K) * N};
    AE_T(weight_scales(ws, ns, 1, amax, mul, sw, s));
    AE_T(launch_pack_fp8(PACK_PLAIN, w, nullptr, nullptr, K, N, N, 0, 0, 1, 1, 64, mul, packed, s));
  }
  hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(256), 0, s, gate, static_cast<size_t>(N), 1.0f);
  AE_T(hipGetLastError());
  AE_T(hipMemsetAsync(y, 0, static_cast<size_t>(M) * N * 4, s));
  // the gated residual epilogue with h = 0 and a unit gate: y = acc * s_x * s_w
  TGemmArgs a = gemm_args(g, codes, sx_row, M, N, K, packed, partial, sw);
  a.h = y;
  a.ldh = N;
  a.gate = gate;
  if (per_column) a.swc = swc;
  AE_T(launch_tgemm(OP_FP8, EPI_RESID, a, g.blocks, s));
  return finish(hipSuccess, s);
}

ae_status aetest_fp8_gate_up(const uint8_t* codes, const float* sx_row, int M, int K, const uint16_t* wg,
                             const uint16_t* wu, int F, float* act, float* sw, int per_column, void* stream) {
  if (!codes || !sx_row || !wg || !wu || !act || !sw || M < 1 || F < 1) return AE_ERR_INVALID_ARGUMENT;
  if (K < 128 || K % 128 || (2 * F) % 128) return AE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int N = 2 * F;
  const TGemmPlan g = plan_tgemm(M, N, K, tgemm_kc(OP_FP8), kTargetBlocks);
  Scratch sc;
  uint4* packed = sc.get<uint4>(static_cast<size_t>(K) * N);
  unsigned* amax = sc.get<unsigned>(8);
  float* mul = sc.get<float>(8);
  float* rowmax = sc.get<float>(static_cast<size_t>(g.n_tiles) * M * 4);
  float* partial = sc.get<float>(tgemm_partial_floats(g) * 4);
  float* cmul = sc.get<float>(static_cast<size_t>(N) * 4);
  float* swc = sc.get<float>(static_cast<size_t>(N) * 4);
  AE_T(sc.err);
  if (per_column) {  // sw: [gate columns | up columns]
    AE_T(launch_fp8_col_scales(wg, K, F, F, cmul, sw, s));
    AE_T(launch_fp8_col_scales(wu, K, F, F, cmul + F, sw + F, s));
    AE_T(launch_pack_fp8(PACK_GU, wg, wu, nullptr, K, N, F, F, 0, 1, 1, 64, cmul, packed, s, cmul, cmul + F));
    AE_T(launch_pack_col_scales(PACK_GU, sw, sw + F, nullptr, N, 1, 1, 64, swc, s));
  } else {
    const uint16_t* ws[2] = {wg, wu};
    const size_t ns[2] = {static_cast<size_t>(K) * F, static_cast<size_t>(K) * F};
    AE_T(weight_scales(ws, ns, 2, amax, mul, sw, s));
    AE_T(launch_pack_fp8(PACK_GU, wg, wu, nullptr, K, N, F, F, 0, 1, 1, 64, mul, packed, s));
  }
  TGemmArgs a = gemm_args(g, codes, sx_row, M, N, K, packed, partial, sw);
  a.out = act;
  a.ldo = F;
  a.rowmax = rowmax;
  a.ldp = M;
  if (per_column) a.swc = swc;
  AE_T(launch_tgemm(OP_FP8, EPI_GELU, a, g.blocks, s));
  return finish(hipSuccess, s);
}

ae_status aetest_fp8_qkv(const uint8_t* codes, const float* sx_row, int M, int K, const uint16_t* wq,
                         const uint16_t* wk, const uint16_t* wv, int Hq, int Hkv, int dh, float* q, float* k,
                         float* v, float* sw, int per_column, void* stream) {
  if (!codes || !sx_row || !wq || !wk || !wv || !q || !k || !v || !sw || M < 1 || Hq < 1 || Hkv < 1)
    return AE_ERR_INVALID_ARGUMENT;
  const int qdim = Hq * dh, kvdim = Hkv * dh, N = qdim + 2 * kvdim;
  if (dh != 64 && dh != 128 && dh != 256) return AE_ERR_UNSUPPORTED;
  if (K < 128 || K % 128 || N % 128) return AE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int S_max = (M + 63) / 64 * 64;
  const TGemmPlan g = plan_tgemm(M, N, K, tgemm_kc(OP_FP8), kTargetBlocks);
  Scratch sc;
  uint4* packed = sc.get<uint4>(static_cast<size_t>(K) * N);
  unsigned* amax = sc.get<unsigned>(12);
  float* mul = sc.get<float>(12);
  float* partial = sc.get<float>(tgemm_partial_floats(g) * 4);
  bf16_t* qb = sc.get<bf16_t>(static_cast<size_t>(M) * qdim * 2);
  bf16_t* kc = sc.get<bf16_t>(static_cast<size_t>(Hkv) * S_max * dh * 2);
  bf16_t* vc = sc.get<bf16_t>(static_cast<size_t>(Hkv) * S_max * dh * 2);
  int* nvalid = sc.get<int>(4);
  float* cosb = sc.get<float>(static_cast<size_t>(M) * (dh / 2) * 4);
  float* sinb = sc.get<float>(static_cast<size_t>(M) * (dh / 2) * 4);
  float* cmul = sc.get<float>(static_cast<size_t>(N) * 4);
  float* swc = sc.get<float>(static_cast<size_t>(N) * 4);
  AE_T(sc.err);
  if (per_column) {  // sw: [q columns | k columns | v columns]
    float *sq = sw, *sk = sw + qdim, *sv = sw + qdim + kvdim;
    AE_T(launch_fp8_col_scales(wq, K, qdim, qdim, cmul, sq, s));
    AE_T(launch_fp8_col_scales(wk, K, kvdim, kvdim, cmul + qdim, sk, s));
    AE_T(launch_fp8_col_scales(wv, K, kvdim, kvdim, cmul + qdim + kvdim, sv, s));
    AE_T(launch_pack_fp8(PACK_QKV, wq, wk, wv, K, N, qdim, kvdim, kvdim, Hq, Hkv, dh, cmul, packed, s, cmul,
                         cmul + qdim, cmul + qdim + kvdim));
    AE_T(launch_pack_col_scales(PACK_QKV, sq, sk, sv, N, Hq, Hkv, dh, swc, s));
  } else {
    const uint16_t* ws[3] = {wq, wk, wv};
    const size_t ns[3] = {static_cast<size_t>(K) * qdim, static_cast<size_t>(K) * kvdim,
                          static_cast<size_t>(K) * kvdim};
    AE_T(weight_scales(ws, ns, 3, amax, mul, sw, s));
    AE_T(launch_pack_fp8(PACK_QKV, wq, wk, wv, K, N, qdim, kvdim, kvdim, Hq, Hkv, dh, mul, packed, s));
  }
  AE_T(hipMemsetAsync(nvalid, 0, 4, s));
  AE_T(hipMemsetAsync(sinb, 0, static_cast<size_t>(M) * (dh / 2) * 4, s));
  hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(256), 0, s, cosb, static_cast<size_t>(M) * (dh / 2), 1.0f);
  AE_T(hipGetLastError());
  TGemmArgs a = gemm_args(g, codes, sx_row, M, N, K, packed, partial, sw);
  a.q = qb;
  a.ldq = qdim;
  a.kcache = kc;
  a.vtcache = vc;
  a.n_valid = nvalid;
  a.rope_cos = cosb;
  a.rope_sin = sinb;
  a.T = M; a.Hq = Hq; a.Hkv = Hkv; a.dh = dh; a.S_max = S_max;
  if (per_column) a.swc = swc;
  AE_T(launch_tgemm(OP_FP8, EPI_QKV, a, g.blocks, s));
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(256), dim3(256), 0, s, qb, static_cast<size_t>(M) * qdim, q);
  hipLaunchKernelGGL(unpack_cache_kernel, dim3(256), dim3(256), 0, s, kc, M, Hkv, dh, S_max, 0, k);
  hipLaunchKernelGGL(unpack_cache_kernel, dim3(256), dim3(256), 0, s, vc, M, Hkv, dh, S_max, 1, v);
  AE_T(hipGetLastError());
  return finish(hipSuccess, s);
}

}  // extern "C"
