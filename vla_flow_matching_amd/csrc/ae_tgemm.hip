// Batched projection GEMMs (many action rows: B * T > 64): Y = A . W on the
// MFMA units with BM x 128 output tiles (BM = 32 rows: many small tiles in
// flight, K split only where they cannot fill the GPU) staged through LDS,
// for bf16
// operands and for the fp8 e4m3 variant of the QKV / gate-up / down
// projections (MolmoBot PR, Part 3: per-tensor dynamic fp8, amax -> cast ->
// scaled matmul; LoongForge blog, section 7: inputs and weights quantised,
// the product restored with both scales).
//
// Around the GEMM:
// * rownorm_kernel forms, for the fp8 inputs, the per-row r and max |u| of
//   the adaRMS input u = h * r * (1 + scale) + shift (LoongForge blog,
//   section 2) that the request-wide scale needs (the bf16 path applies the
//   norm after the product instead).
// * quant_kernel turns fp32 rows (u recomputed bit-identically, or the
//   gelu * up activations) into e4m3 codes with the per-request scale
//   amax / 448, deciding every code in fp32.
// * The GEMM epilogues are the expert's: RoPE + q / K / V^T scatter, gelu of
//   the gate half times the up half, and the gated residual h += gate * y.
//   In fp8 mode y = acc * s_x(request) * s_w(tensor) first.
//
// A is row-major [M][lda] in the operand type; W is pre-packed in fragment
// order so that one 128-byte k-chunk of a 16-column group is 2 KiB
// contiguous.  Rows beyond M read a clamped (valid) row and are never
// stored.  Split-K partials are summed in split order by a second kernel
// (one workgroup per 16 rows of a tile), so results do not depend on
// scheduling.
#include "ae_device.h"
#include "ae_kernels.h"

namespace ae {

namespace {

constexpr int kTT = 256;     // threads per GEMM workgroup (4 waves, 32 columns each)
constexpr int kBN = 128;     // tile columns
constexpr int kXcd = 8;
constexpr int kMaxSplit = 8;    // K splits of one tile at most

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// OCP e4m3fn encoding (round to nearest even, saturating at +-448,
// subnormal step 2^-9): the code of the e4m3 value nearest to v.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {
    // below the smallest normal 2^-6 the spacing is 2^-9: code = a / 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    // keep 3 fraction bits of the fp32 value, ties to even
    const uint32_t ab = __float_as_uint(a);
    uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) & 0xFFF00000u;
    if (__uint_as_float(r) > 448.0f) r = __float_as_uint(448.0f);
    code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  }
  return sign | code;
}

// 16 fp32 values -> 16 codes (one uint4), value i in byte i.
__device__ __forceinline__ uint4 e4m3_pack16(const float* v, float mul) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = e4m3_code(v[4 * j] * mul) | (e4m3_code(v[4 * j + 1] * mul) << 8) |
           (e4m3_code(v[4 * j + 2] * mul) << 16) | (e4m3_code(v[4 * j + 3] * mul) << 24);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// fp8 scale pair from an amax: (448 / a, a / 448) with a = max(amax, 1e-12),
// both divisions correctly rounded fp32.
__device__ __forceinline__ float fp8_mul(float amax) { return 448.0f / fmaxf(amax, 1e-12f); }
__device__ __forceinline__ float fp8_scale(float amax) { return fmaxf(amax, 1e-12f) / 448.0f; }

// adaRMS of one element; the one expression both the norm and the quantiser
// evaluate, so the fp32 u they see is the same value.
__device__ __forceinline__ float ada(float h, float r, float sc, float sh) {
  return h * r * (1.0f + sc) + sh;
}

// ---------------------------------------------------------------------------
// Sum / max over a 256-thread workgroup (lane swaps within each wave, then
// the four wave results through LDS); every thread gets the result.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_sum(float v, float* s_red) {
  v = wave_sum(v);
  __syncthreads();  // (s_red may still be read by a previous call)
  if (threadIdx.x % kWave == 0) s_red[threadIdx.x / kWave] = v;
  __syncthreads();
  return (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

__device__ __forceinline__ float block_max(float v, float* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if (threadIdx.x % kWave == 0) s_red[threadIdx.x / kWave] = v;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

// ---------------------------------------------------------------------------
// Row norm of the fp8 inputs: one 256-thread workgroup per row (all of a
// row's loads in flight at once): r[row] = 1 / rms(h row) and rowmax[row] =
// max_k |u|, u = adaRMS(h).  D <= 4 * 256 * kNormPer.
// ---------------------------------------------------------------------------
constexpr int kNormPer = 4;  // float4 per thread held across the two passes (D <= 4096)

__global__ __launch_bounds__(256) void rownorm_kernel(const float* __restrict__ h, int M, int D,
                                                      const float* __restrict__ scale,
                                                      const float* __restrict__ shift, float eps,
                                                      float* __restrict__ r_out,
                                                      float* __restrict__ rowmax) {
  __shared__ float s_red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float4* hr = reinterpret_cast<const float4*>(h + static_cast<size_t>(row) * D);
  const int n4 = D / 4;
  float4 v[kNormPer];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int i = tid + 256 * j;
    v[j] = i < n4 ? hr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  ss = block_sum(ss, s_red);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  const float4* sc4 = reinterpret_cast<const float4*>(scale);
  const float4* sh4 = reinterpret_cast<const float4*>(shift);
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int i = tid + 256 * j;
    if (i >= n4) break;
    const float4 s = sc4[i], b = sh4[i];
    const float o0 = ada(v[j].x, r, s.x, b.x), o1 = ada(v[j].y, r, s.y, b.y);
    const float o2 = ada(v[j].z, r, s.z, b.z), o3 = ada(v[j].w, r, s.w, b.w);
    mx = fmaxf(fmaxf(mx, fmaxf(fabsf(o0), fabsf(o1))), fmaxf(fabsf(o2), fabsf(o3)));
  }
  mx = block_max(mx, s_red);
  if (tid == 0) {
    r_out[row] = r;
    rowmax[row] = mx;
  }
}

// ---------------------------------------------------------------------------
// Quantiser: one 256-thread workgroup per row.  The request's amax is the
// max of rowmax[p][rows of the request] over the n_part partial columns; the
// row is then coded with 448 / amax.  src == nullptr: the row is u
// recomputed from h, r and the modulation; otherwise src [M][K] fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_kernel(const float* __restrict__ src,
                                                    const float* __restrict__ h,
                                                    const float* __restrict__ r_in,
                                                    const float* __restrict__ scale,
                                                    const float* __restrict__ shift, int M, int K,
                                                    int T, const float* __restrict__ rowmax,
                                                    int n_part, int ldp, uint8_t* __restrict__ codes,
                                                    float* __restrict__ sx_row) {
  __shared__ float s_red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int r0 = (row / T) * T;
  // one load per thread, or (many partial columns) 16 per thread in flight
  // per pass, clamped and masked at use
  float mx = 0.0f;
  const int n = n_part * T;
  if (n <= 256) {
    if (tid < n) mx = rowmax[static_cast<size_t>(tid / T) * ldp + r0 + tid % T];
  } else for (int i0 = 0; i0 < n; i0 += 16 * 256) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = min(i0 + tid + 256 * j, n - 1);
      v[j] = rowmax[static_cast<size_t>(i / T) * ldp + r0 + i % T];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (i0 + tid + 256 * j < n) mx = fmaxf(mx, v[j]);
  }
  mx = block_max(mx, s_red);
  const float mul = fp8_mul(mx);
  if (tid == 0) sx_row[row] = fp8_scale(mx);
  const int n16 = K / 16;
  uint4* out = reinterpret_cast<uint4*>(codes + static_cast<size_t>(row) * K);
  for (int i = tid; i < n16; i += 256) {
    float v[16];
    if (src) {
      const float4* s4 = reinterpret_cast<const float4*>(src + static_cast<size_t>(row) * K) + 4 * i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = s4[j];
        v[4 * j] = x.x; v[4 * j + 1] = x.y; v[4 * j + 2] = x.z; v[4 * j + 3] = x.w;
      }
    } else {
      const float r = r_in[row];
      const float4* h4 = reinterpret_cast<const float4*>(h + static_cast<size_t>(row) * K) + 4 * i;
      const float4* c4 = reinterpret_cast<const float4*>(scale) + 4 * i;
      const float4* b4 = reinterpret_cast<const float4*>(shift) + 4 * i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = h4[j], s = c4[j], b = b4[j];
        v[4 * j] = ada(x.x, r, s.x, b.x);
        v[4 * j + 1] = ada(x.y, r, s.y, b.y);
        v[4 * j + 2] = ada(x.z, r, s.z, b.z);
        v[4 * j + 3] = ada(x.w, r, s.w, b.w);
      }
    }
    out[i] = e4m3_pack16(v, mul);
  }
}

// ---------------------------------------------------------------------------
// The tiled GEMM.
//
// Operand chunk in LDS (16 KiB): [8 groups of 16 rows or columns][2 slots]
// [64 lanes][16 bytes].  bf16: slot s is k-fragment s of the 64-wide
// chunk, lane l holds row l%16, k = 32s + 8(l/16) .. +7.  fp8: the chunk is
// one 128-wide k-fragment of the 16x16x128 MFMA; lane l holds row l%16 and
// k = 32(l/16) .. +31, slot s its bytes 16s .. 16s+15.  A and B use the same
// map, so the hardware pairs matching k on both sides.
// ---------------------------------------------------------------------------
template <int OP> struct TOp;
template <> struct TOp<OP_BF16> {
  static constexpr int KC = 64;  // k per chunk
  static __device__ __forceinline__ int slot_lane(int kc, int r16, int& lane) {
    lane = r16 + 16 * (kc & 3);
    return kc >> 2;
  }
};
template <> struct TOp<OP_FP8> {
  static constexpr int KC = 128;
  static __device__ __forceinline__ int slot_lane(int kc, int r16, int& lane) {
    lane = r16 + 16 * (kc >> 1);
    return kc & 1;
  }
};

__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
  const i32x8 a = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                   static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                   static_cast<int>(a1.z), static_cast<int>(a1.w)};
  const i32x8 b = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                   static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                   static_cast<int>(b1.z), static_cast<int>(b1.w)};
  // formats 0/0: e4m3 on both sides; scales 127 = 2^0 (no block scaling)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Position of A-fragment lane l of slot s inside its 1 KiB LDS block.  The
// staging threads write 16-byte pieces of two rows x eight k-pieces per 16
// lanes; XOR-ing the row bits with (k group, slot) spreads those 16 writes
// over all 64 banks, and a reading wave's 16-lane groups still cover 16
// distinct bank quads.
__device__ __forceinline__ int swz(int l, int s) {
  const int q = l >> 4;
  return 16 * q + ((l & 15) ^ ((2 * q + 8 * s) & 15));
}

// One chunk times the wave's BM x 32 block of the tile (RT = BM / 16 row
// tiles x two 16-column groups): A fragments from the LDS stage, B fragments
// (two 16-column groups x two slots) from registers.
template <int OP, int RT>
__device__ __forceinline__ void tg_compute(const uint4* A, const u32x4 (&B)[2][2], int lane,
                                           f32x4 (&acc)[RT][2]) {
  if (OP == OP_BF16) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 a[RT];
#pragma unroll
      for (int i = 0; i < RT; ++i) a[i] = A[(i * 2 + s) * kWave + swz(lane, s)];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(a[i], __builtin_bit_cast(uint4, B[j][s]), acc[i][j]);
    }
  } else {
    uint4 a[RT][2];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s) a[i][s] = A[(i * 2 + s) * kWave + swz(lane, s)];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = mfma_fp8(a[i][0], a[i][1], __builtin_bit_cast(uint4, B[j][0]),
                             __builtin_bit_cast(uint4, B[j][1]), acc[i][j]);
  }
}

// Tile decode.  Units (n-tile, m-tile, K split) in that order are cut into
// eight equal contiguous ranges, one per XCD (workgroups are dealt to the 8
// XCDs round-robin), so the m-tiles of an n-tile share one L2 (or two, where
// a range boundary falls inside them) and every XCD gets the same number of
// units whatever the n-tile count (dealing whole n-tiles to XCDs left XCDs
// idle below 8 n-tiles and unbalanced at 20).
__device__ __forceinline__ bool tile_of(int bid, int n_tiles, int m_tiles, int ksplit, int& nt,
                                        int& mt, int& s) {
  const int units = n_tiles * m_tiles * ksplit;
  const int per_xcd = (units + kXcd - 1) / kXcd;
  const int li = bid / kXcd;
  const int u = (bid % kXcd) * per_xcd + li;
  if (li >= per_xcd || u >= units) return false;
  s = u % ksplit;
  mt = (u / ksplit) % m_tiles;
  nt = u / (ksplit * m_tiles);
  return true;
}

// The GEMM epilogues on rows [m0, m0 + rows) of n-tile nt, the finished
// values in s_y (row-major, relative to m0); wave w takes rows w, w + 4, ...
// s_r[row] = 1 / rms of row m0 + row from its 64-column partial sums of
// squares over K columns.  TPR threads per row each add every TPR-th partial
// (a fixed, unrolled set of loads, all in flight at once: norm_issue) and the
// row's threads combine with lane swaps (norm_finish); rows <= kTT / TPR,
// partials <= 64.
template <int TPR>
struct RowNorm {
  static_assert(TPR == 2 || TPR == 4 || TPR == 16, "threads per row (a quad, or a whole 16-lane row)");
  static constexpr int kPer = 64 / TPR;
  float v[kPer];

  __device__ __forceinline__ void issue(const TGemmArgs& p, int m0, int rows) {
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
    const int m = m0 + min(row, rows - 1);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = min(part + TPR * j, p.ssq_tiles - 1);
      v[j] = p.ssq[static_cast<size_t>(q) * p.ldssq + m];
    }
  }
  // (the caller synchronises before reading s_r)
  __device__ __forceinline__ void finish(const TGemmArgs& p, int rows, float* s_r) const {
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (part + TPR * j < p.ssq_tiles) t += v[j];
    t += xor1_swap(t);
    if (TPR >= 4) t += xor2_swap(t);
    if (TPR == 16) {  // the four quad sums of the 16-lane row
      t += row_ror<4>(t);
      t += row_ror<8>(t);
    }
    if (part == 0 && row < rows) s_r[row] = 1.0f / sqrtf(t / static_cast<float>(p.K) + p.eps);
  }
};

// (s_r: LDS scratch of >= rows floats for the norm after the product.)
// Rows go in batches of kEB per wave: a batch's loads are all issued before
// any of its stores, and per-column constants are loaded once, so a row
// never waits for its own round trip behind the previous row's stores.
constexpr int kEB = 8;

// (R_READY: s_r was filled before the product)
template <int OP, int EPI, int TPR, bool R_READY>
__device__ __forceinline__ void tg_epilogue(const TGemmArgs& p, int nt, int m0, int rows,
                                            float (*s_y)[kBN + 1], float* s_r) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bool post_norm = OP == OP_BF16 && EPI != EPI_RESID && p.bias != nullptr;
  if (post_norm && !R_READY) {
    RowNorm<TPR> rn;
    rn.issue(p, m0, rows);
    rn.finish(p, rows, s_r);
    __syncthreads();
  }
  // column pair structure of the packed layout: packed column pc of this
  // tile is pair P = 4 nt + pc / 32, half pc / 16 % 2, index pc % 16
  const int pr = lane / 16, jj = lane % 16;
  float bias_a = 0.0f, bias_b = 0.0f;
  if (post_norm) {
    bias_a = p.bias[nt * kBN + 32 * pr + jj];
    bias_b = p.bias[nt * kBN + 32 * pr + 16 + jj];
  }
  if (EPI == EPI_RESID) {
    // h += gate * y (fp8: y = acc * s_x * s_w); two columns per lane; then,
    // for a norm applied after the next product, the row sums of squares
    // per 64 columns and the modulated bf16 shadow
    float gt[2], ns[2], cw[2];
    const bool colw = OP == OP_FP8 && p.swc != nullptr;  // row-wise: a weight scale per column
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const int n = nt * kBN + 64 * hc + lane;
      gt[hc] = p.gate[n];
      ns[hc] = p.nsc ? 1.0f + p.nsc[n] : 0.0f;
      cw[hc] = colw ? p.swc[n] : 1.0f;
    }
    for (int rb = wave; rb < rows; rb += 4 * kEB) {
      float hv[kEB][2], sxv[kEB];
#pragma unroll
      for (int i = 0; i < kEB; ++i) {
        const int m = m0 + min(rb + 4 * i, rows - 1);
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) hv[i][hc] = p.h[static_cast<size_t>(m) * p.ldh + nt * kBN + 64 * hc + lane];
        sxv[i] = OP == OP_FP8 ? (colw ? p.sx_row[m] : p.sx_row[m] * p.sw[0]) : 1.0f;
      }
#pragma unroll
      for (int i = 0; i < kEB; ++i) {
        const int row = rb + 4 * i;
        if (row >= rows) break;
        const int m = m0 + row;
        float sq[2];
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
          const int n = nt * kBN + 64 * hc + lane;
          const float y = colw ? (s_y[row][64 * hc + lane] * sxv[i]) * cw[hc] : s_y[row][64 * hc + lane] * sxv[i];
          const float hn = hv[i][hc] + gt[hc] * y;
          p.h[static_cast<size_t>(m) * p.ldh + n] = hn;
          sq[hc] = hn * hn;
          if (p.nsc) p.ha[static_cast<size_t>(m) * p.ldh + n] = f2bf(hn * ns[hc]);
        }
        if (p.ssq) {
#pragma unroll
          for (int hc = 0; hc < 2; ++hc) {
            const float t = wave_sum(sq[hc]);
            if (lane == 0) p.ssq[static_cast<size_t>(2 * nt + hc) * p.ldssq + m] = t;
          }
        }
      }
    }
  } else if (EPI == EPI_GELU) {
    // lanes: 64 = 4 pairs x 16; gate half at 32 pr + jj, up half at +16
    const int f = (4 * nt + pr) * 16 + jj;
    float sw0 = OP == OP_FP8 ? p.sw[0] : 1.0f, sw1 = OP == OP_FP8 ? p.sw[1] : 1.0f;
    if (OP == OP_FP8 && p.swc) {  // row-wise: the gate column's and the up column's own scales
      sw0 = p.swc[nt * kBN + 32 * pr + jj];
      sw1 = p.swc[nt * kBN + 32 * pr + 16 + jj];
    }
    for (int rb = wave; rb < rows; rb += 4 * kEB) {
      float sxv[kEB];
#pragma unroll
      for (int i = 0; i < kEB; ++i) sxv[i] = OP == OP_FP8 ? p.sx_row[m0 + min(rb + 4 * i, rows - 1)] : 1.0f;
#pragma unroll
      for (int i = 0; i < kEB; ++i) {
        const int row = rb + 4 * i;
        if (row >= rows) break;
        const int m = m0 + row;
        float g = s_y[row][32 * pr + jj], u = s_y[row][32 * pr + 16 + jj];
        if (post_norm) {
          const float r = s_r[row];
          g = g * r + bias_a;
          u = u * r + bias_b;
        }
        if (OP == OP_FP8) {
          g = g * (sxv[i] * sw0);
          u = u * (sxv[i] * sw1);
        }
        const float a = gelu_tanh(g) * u;
        if (OP == OP_FP8) {
          static_cast<float*>(p.out)[static_cast<size_t>(m) * p.ldo + f] = a;
          float mx = fabsf(a);
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
          if (lane == 0) p.rowmax[static_cast<size_t>(nt) * p.ldp + m] = mx;
        } else {
          static_cast<bf16_t*>(p.out)[static_cast<size_t>(m) * p.ldo + f] = f2bf(a);
        }
      }
    }
  } else {  // EPI_QKV
    const int pph = p.dh / 32;
    const int pq = p.Hq * pph, pk = p.Hkv * pph;
    const int half = p.dh / 2;
    int P = 4 * nt + pr;
    size_t lofs = 0;  // (several layers in one product: the caches of this column's layer)
    if (p.ctx_layer_cols > 0) {
      const int ppl = p.ctx_layer_cols / 32;
      const int layer = P / ppl;
      P -= layer * ppl;
      lofs = static_cast<size_t>(layer) * p.ctx_layer_elems;
    }
    int seg, head, pi;
    if (P < pq) { seg = 0; head = P / pph; pi = P % pph; }
    else if (P < pq + pk) { seg = 1; head = (P - pq) / pph; pi = (P - pq) % pph; }
    else { seg = 2; head = (P - pq - pk) / pph; pi = (P - pq - pk) % pph; }
    const int j = 16 * pi + jj;
    // fp8 weight scales of the pair's two columns (per tensor: the segment's)
    float swa = OP == OP_FP8 ? p.sw[seg] : 1.0f, swb = swa;
    if (OP == OP_FP8 && p.swc) {
      swa = p.swc[nt * kBN + 32 * pr + jj];
      swb = p.swc[nt * kBN + 32 * pr + 16 + jj];
    }
    bf16_t* qo = static_cast<bf16_t*>(p.q);
    bf16_t* kc = static_cast<bf16_t*>(p.kcache) + lofs;
    bf16_t* vt = static_cast<bf16_t*>(p.vtcache) + lofs;
    const bool ctx = p.key_map != nullptr;
    if (!ctx && 4 * nt >= pq + pk) {
      // A tile of V columns only (not rotated).  V^T rows are head dims, so
      // lanes (tile column 8 (wave + 4 u) + lane / 8, row 8 q + lane % 8)
      // make each store instruction cover eight columns' runs of eight
      // consecutive keys instead of 64 dims of one key 16 bytes apart.
      const int kr = lane % 8, cl = lane / 8;
      float vb[4], vs[4];
      size_t vhead[4];
      int vd[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = 8 * (wave + 4 * u) + cl;
        const int Pv = 4 * nt + c / 32 - pq - pk;
        vhead[u] = static_cast<size_t>(Pv / pph) * p.S_max * p.dh;
        vd[u] = ((c & 16) ? half : 0) + 16 * (Pv % pph) + c % 16;
        vb[u] = post_norm ? p.bias[nt * kBN + c] : 0.0f;
        vs[u] = OP == OP_FP8 ? (p.swc ? p.swc[nt * kBN + c] : p.sw[2]) : 1.0f;
      }
      constexpr int kQ = 8;  // row groups of 8 (tiles hold at most 64 rows)
      int vkey[kQ], vreq[kQ];
      float vrs[kQ], vsx[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int rc = min(8 * q + kr, rows - 1);
        const int m = m0 + rc;
        vreq[q] = m / p.T;
        vkey[q] = p.n_valid[vreq[q]] + m % p.T;
        vrs[q] = post_norm ? s_r[rc] : 1.0f;
        vsx[q] = OP == OP_FP8 ? p.sx_row[m] : 1.0f;
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (8 * q >= rows) break;
        const int row = 8 * q + kr, rc = min(row, rows - 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = 8 * (wave + 4 * u) + cl;
          float y = s_y[rc][c];
          if (post_norm) y = y * vrs[q] + vb[u];
          if (OP == OP_FP8) y *= vsx[q] * vs[u];
          if (row < rows)
            vt[(static_cast<size_t>(vreq[q]) * p.Hkv) * p.S_max * p.dh + vhead[u] +
               KvLayout<bf16_t>::v_off(vkey[q], vd[u], p.dh)] = f2bf(y);
        }
      }
      return;
    }
    for (int rb = wave; rb < rows; rb += 4 * kEB) {
      float csv[kEB], snv[kEB], sxv[kEB];
      int nvv[kEB];  // the row's cache key
#pragma unroll
      for (int i = 0; i < kEB; ++i) {
        const int m = m0 + min(rb + 4 * i, rows - 1);
        const int req = m / p.T, t = m % p.T;
        if (ctx) {  // a context row: its own key, rotated at that position
          nvv[i] = p.key_map[m];
          const size_t pi2 = static_cast<size_t>(max(nvv[i], 0)) * half + j;
          csv[i] = p.pos_cos[pi2];
          snv[i] = p.pos_sin[pi2];
        } else {
          const size_t ti2 = (static_cast<size_t>(req) * p.T + t) * half + j;
          csv[i] = p.rope_cos[ti2];
          snv[i] = p.rope_sin[ti2];
          nvv[i] = p.n_valid[req] + t;
        }
        sxv[i] = OP == OP_FP8 ? p.sx_row[m] : 1.0f;
      }
#pragma unroll
      for (int i = 0; i < kEB; ++i) {
        const int row = rb + 4 * i;
        if (row >= rows) break;
        const int m = m0 + row;
        const int req = m / p.T;
        float a = s_y[row][32 * pr + jj], b = s_y[row][32 * pr + 16 + jj];
        if (post_norm) {
          const float r = s_r[row];
          a = a * r + bias_a;
          b = b * r + bias_b;
        }
        if (OP == OP_FP8) {
          a *= sxv[i] * swa;
          b *= sxv[i] * swb;
        }
        if (seg < 2) {
          const float ra = a * csv[i] - b * snv[i];
          const float rb2 = b * csv[i] + a * snv[i];
          a = ra;
          b = rb2;
        }
        if (seg == 0) {
          bf16_t* dst = qo + static_cast<size_t>(m) * p.ldq + head * p.dh;
          dst[j] = f2bf(a);
          dst[half + j] = f2bf(b);
        } else {
          const int key = nvv[i];
          if (key < 0) continue;  // an invisible context row: never stored
          const size_t base = static_cast<size_t>(req) * p.Hkv + head;
          using LY = KvLayout<bf16_t>;
          bf16_t* dst = (seg == 1 ? kc : vt) + base * p.S_max * p.dh;
          if (seg == 1) {
            dst[LY::k_off(key, j, p.dh)] = f2bf(a);
            dst[LY::k_off(key, half + j, p.dh)] = f2bf(b);
          } else {
            dst[LY::v_off(key, j, p.dh)] = f2bf(a);
            dst[LY::v_off(key, half + j, p.dh)] = f2bf(b);
          }
        }
      }
    }
  }
}

// threads per row of the row-norm sums (RowNorm): rows <= kTT / TPR
template <int BM>
constexpr int norm_tpr() {
  return BM >= 128 ? 2 : 4;
}

// CPS: K chunks per LDS stage (one barrier per stage).
template <int OP, int EPI, int BM, int CPS>
__global__ __launch_bounds__(kTT, 2) void tgemm_kernel(TGemmArgs p) {
  using O = TOp<OP>;
  constexpr int KC = O::KC;
  constexpr int RT = BM / 16;              // 16-row tiles per wave
  constexpr int NA = BM / 32;              // A staging pieces per thread per chunk
  constexpr int kChunkU4 = BM * 8;         // uint4 per staged A chunk
  constexpr int kStageU4 = CPS * kChunkU4;
  constexpr int kTileU4 = BM * (kBN + 1) / 4 + BM / 4;
  constexpr int kBufU4 = kTileU4 > 2 * kStageU4 ? kTileU4 : 2 * kStageU4;
  // two stages of A chunks; the finished tile reuses the space
  // (+ 1 / rms of the tile's rows past the finished tile)
  __shared__ __attribute__((aligned(16))) uint4 s_buf[kBufU4];
  auto s_y = reinterpret_cast<float (*)[kBN + 1]>(s_buf);
  static_assert(kBufU4 >= 16 * 64, "16 KiB of LDS for a prefetch workgroup");

  if (static_cast<int>(blockIdx.x) >= p.main_blocks) {  // a prefetch workgroup
    prefetch_ranges<kTT, 16>(p.pf, p.pf_n4, 2, blockIdx.x - p.main_blocks, p.pf_blocks,
                             static_cast<uint32_t>(reinterpret_cast<size_t>((lds_void_t*)(s_buf))));
    return;
  }
  int nt, mt, ks;
  if (!tile_of(blockIdx.x, p.n_tiles, p.m_tiles, p.ksplit, nt, mt, ks)) return;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int m0 = mt * BM;
  const int rows = min(BM, p.M - m0);
  const int n_chunks = p.K / KC;
  // stage indices (CPS chunks each) of this split
  const int n_stages = n_chunks / CPS;
  const int c0 = static_cast<int>((static_cast<long long>(ks) * n_stages) / p.ksplit);
  const int c1 = static_cast<int>((static_cast<long long>(ks + 1) * n_stages) / p.ksplit);
  // the rows' 1 / rms for a norm after the product (into LDS past the
  // finished tile): loads issued after the first chunk's, summed after the
  // K loop
  float* s_r = reinterpret_cast<float*>(s_buf) + BM * (kBN + 1);
  const bool norm_here = OP == OP_BF16 && EPI != EPI_RESID && p.bias != nullptr && p.ksplit == 1;
  RowNorm<norm_tpr<BM>()> rn;

  // A staging map: item i = tid + 256 j: row i/8, 16-byte column i%8.
  const uint8_t* Ab = static_cast<const uint8_t*>(p.A);
  if (p.ctx_layer_cols > 0)  // (several layers in one product: this tile's layer's rows)
    Ab += static_cast<size_t>((nt * kBN) / p.ctx_layer_cols) * p.a_layer_bytes;
  uint32_t a_off[NA];
  int a_lds[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int i = tid + kTT * j;
    const int row = i >> 3, kc = i & 7;
    const int grow = min(m0 + row, p.M - 1);
    a_off[j] = static_cast<uint32_t>(grow) * static_cast<uint32_t>(p.lda_bytes) + 16u * kc;
    int ln;
    const int slot = O::slot_lane(kc, row & 15, ln);
    a_lds[j] = ((row >> 4) * 2 + slot) * kWave + swz(ln, slot);
  }
  // B fragments go straight to registers: wave w reads the 2 KiB chunk of
  // each of its two 16-column groups (32 w .. 32 w + 31 of the tile) itself,
  // so every weight byte is read once per tile and only A passes through LDS.
  const u32x4* Wv = reinterpret_cast<const u32x4*>(p.W) +
                    (static_cast<size_t>(nt) * 8 + 2 * wave) * n_chunks * 128 + lane;
  u32x4* sv = reinterpret_cast<u32x4*>(s_buf);

  struct AStage {
    u32x4 a[CPS][NA];
  };
  struct BStage {
    u32x4 b[CPS][2][2];
  };
  // (c: a stage index, chunks CPS c .. CPS c + CPS - 1)
#define TG_LOAD_A(R, c)                                                            \
  do {                                                                             \
    _Pragma("unroll") for (int q_ = 0; q_ < CPS; ++q_) {                           \
      const uint32_t co_ = static_cast<uint32_t>(CPS * (c) + q_) * 128u;           \
      _Pragma("unroll") for (int j_ = 0; j_ < NA; ++j_)                            \
        R.a[q_][j_] = *reinterpret_cast<const u32x4*>(Ab + a_off[j_] + co_);       \
    }                                                                              \
  } while (0)
#define TG_LOAD_B(R, c)                                                            \
  do {                                                                             \
    _Pragma("unroll") for (int q_ = 0; q_ < CPS; ++q_)                             \
      _Pragma("unroll") for (int j_ = 0; j_ < 2; ++j_)                             \
        _Pragma("unroll") for (int s_ = 0; s_ < 2; ++s_)                           \
          R.b[q_][j_][s_] = Wv[(static_cast<size_t>(j_) * n_chunks + CPS * (c) + q_) * 128 + s_ * 64]; \
  } while (0)
#define TG_STORE_A(R, st)                                                          \
  do {                                                                             \
    u32x4* sa_ = sv + (st) * kStageU4;                                             \
    _Pragma("unroll") for (int q_ = 0; q_ < CPS; ++q_)                             \
      _Pragma("unroll") for (int j_ = 0; j_ < NA; ++j_)                            \
        sa_[q_ * kChunkU4 + a_lds[j_]] = R.a[q_][j_];                              \
  } while (0)
#define TG_COMPUTE(st, RB)                                                         \
  do {                                                                             \
    _Pragma("unroll") for (int q_ = 0; q_ < CPS; ++q_)                             \
      tg_compute<OP, RT>(s_buf + (st) * kStageU4 + q_ * kChunkU4, RB[q_], lane, acc); \
  } while (0)

  f32x4 acc[RT][2];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Iteration c: LDS stage c%2 holds A(c), registers hold B(c); A(c+1) and
  // B(c+1) are in flight and A(c+2) is issued.  Every split holds at least
  // one chunk (plan_tgemm); chunk indices past the split are clamped (the
  // tail re-loads its last chunk into a stage nobody reads).
  AStage a0, a1;
  BStage b0, b1;
  TG_LOAD_A(a0, c0);
  TG_LOAD_B(b0, c0);
  TG_STORE_A(a0, 0);
  TG_LOAD_A(a1, min(c0 + 1, c1 - 1));
  if (norm_here) rn.issue(p, m0, rows);
  __syncthreads();
  int c = c0;
  // (the scheduling barriers keep each chunk's global loads ahead of the
  // multiply instead of letting them sink to their uses)
  for (; c + 1 < c1; c += 2) {
    TG_LOAD_B(b1, c + 1);
    TG_LOAD_A(a0, min(c + 2, c1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    TG_COMPUTE(0, b0.b);
    TG_STORE_A(a1, 1);
    __syncthreads();
    TG_LOAD_B(b0, min(c + 2, c1 - 1));
    TG_LOAD_A(a1, min(c + 3, c1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    TG_COMPUTE(1, b1.b);
    TG_STORE_A(a0, 0);
    __syncthreads();
  }
  if (c < c1) {
    TG_COMPUTE(0, b0.b);  // odd stage count: the last stage sits in stage buffer 0
    __syncthreads();      // every wave is done with the stages before s_y reuses them
  }
  if (norm_here) rn.finish(p, rows, s_r);  // (read after the s_y barrier below)
#undef TG_LOAD_A
#undef TG_LOAD_B
#undef TG_STORE_A
#undef TG_COMPUTE

  // accumulators -> LDS tile (row-major)
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s_y[16 * i + 4 * (lane / 16) + e][32 * wave + 16 * j + lane % 16] = acc[i][j][e];
  __syncthreads();

  if (p.ksplit > 1) {
    // this split's rows of the tile -> partial scratch; the reduce kernel
    // that follows sums the splits in order and applies the epilogue
    float* part = p.partial + (static_cast<size_t>(nt * p.m_tiles + mt) * p.ksplit + ks) * (BM * kBN);
    const int n4 = rows * (kBN / 4);
    for (int i = tid; i < n4; i += kTT) {
      const int r = i / (kBN / 4), c4 = 4 * (i % (kBN / 4));
      *reinterpret_cast<float4*>(part + r * kBN + c4) =
          make_float4(s_y[r][c4], s_y[r][c4 + 1], s_y[r][c4 + 2], s_y[r][c4 + 3]);
    }
    return;
  }
  tg_epilogue<OP, EPI, norm_tpr<BM>(), true>(p, nt, m0, rows, s_y, s_r);
}

// Sum of a tile's K-split partials for RR rows (in split order), then the
// epilogue of those rows.  One workgroup per (tile, RR-row slice): 4-row
// slices for products of at most 64 rows (one request: 16-50 rows) and
// wherever 16-row slices would leave CUs idle, so the reduction spreads over
// four times the workgroups, each with a quarter of the partial bytes in
// flight; 16-row slices otherwise.
constexpr int kRedSlicesWanted = 256;  // 16-row slices that keep every CU busy

template <int OP, int EPI, int BM, int RR>
__global__ __launch_bounds__(kTT) void tgemm_reduce_kernel(TGemmArgs p) {
  static_assert(RR == 16 || RR == 4, "16- or 4-row slices");
  __shared__ float s_y[RR][kBN + 1];
  __shared__ float s_r[16];
  constexpr int slices = BM / RR;
  constexpr int NV = RR * kBN / 4;              // float4 of the slice
  constexpr int U = (NV + kTT - 1) / kTT;       // per thread
  const int tile = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int nt = tile / p.m_tiles, mt = tile % p.m_tiles;
  const int m0 = mt * BM + sl * RR;
  const int rows = min(RR, p.M - m0);
  if (rows <= 0) return;
  const int tid = threadIdx.x;
  const float* part = p.partial + static_cast<size_t>(tile) * p.ksplit * (BM * kBN) + sl * RR * kBN;
  // every split of the thread's float4s in flight together
  float4 v[U][kMaxSplit];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = min(tid + u * kTT, NV - 1);
    const int r = min(i / (kBN / 4), rows - 1), c4 = 4 * (i % (kBN / 4));
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
      v[u][q] = *reinterpret_cast<const float4*>(part + static_cast<size_t>(min(q, p.ksplit - 1)) * (BM * kBN) +
                                                 r * kBN + c4);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = tid + u * kTT;
    if (i >= NV) continue;
    const int r = i / (kBN / 4), c4 = 4 * (i % (kBN / 4));
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
      if (q < p.ksplit) {
        t.x += v[u][q].x; t.y += v[u][q].y; t.z += v[u][q].z; t.w += v[u][q].w;
      }
    s_y[r][c4] = t.x; s_y[r][c4 + 1] = t.y; s_y[r][c4 + 2] = t.z; s_y[r][c4 + 3] = t.w;
  }
  __syncthreads();
  // (the post-norm row scales: 16 threads per row; past `rows` they repeat
  // the last row and store nothing)
  tg_epilogue<OP, EPI, 16, false>(p, nt, m0, rows, s_y, s_r);
}

// ---------------------------------------------------------------------------
// fp8 weights: per-tensor amax, then codes packed in the GEMM's chunk order
// [N/16][K/128][2 slots][64 lanes][16 B] (columns reordered like the bf16
// packing: PACK_QKV rope pairs, PACK_GU gate/up pairs).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void amax_kernel(const bf16_t* __restrict__ w, size_t n,
                                                   unsigned* __restrict__ out) {
  float mx = 0.0f;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    mx = fmaxf(mx, fabsf(bf2f(w[i])));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  // non-negative floats order like their bit patterns
  if (threadIdx.x % kWave == 0) atomicMax(out, __float_as_uint(mx));
}

__global__ void scales_kernel(const unsigned* __restrict__ amax_bits, int n, float* __restrict__ mul,
                              float* __restrict__ scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float a = __uint_as_float(amax_bits[i]);
    mul[i] = fp8_mul(a);
    scale[i] = fp8_scale(a);
  }
}

// The logical source (0, 1, 2) and column of packed column pc: PACK_PLAIN
// keeps the order; PACK_GU interleaves 16-column runs of gate and up;
// PACK_QKV puts the two halves of each RoPE pair of q, then k, then v side by
// side (16 + 16 columns).
__device__ __forceinline__ void packed_source(int mode, int pc, int Hq, int Hkv, int dh, int& which, int& col) {
  if (mode == PACK_PLAIN) {
    which = 0;
    col = pc;
    return;
  }
  const int P = pc / 32, hf = (pc / 16) % 2, jj = pc % 16;
  if (mode == PACK_GU) {
    which = hf;
    col = 16 * P + jj;
    return;
  }
  const int pph = dh / 32, pq = Hq * pph, pk = Hkv * pph;
  int head, pi;
  if (P < pq) { which = 0; head = P / pph; pi = P % pph; }
  else if (P < pq + pk) { which = 1; head = (P - pq) / pph; pi = (P - pq) % pph; }
  else { which = 2; head = (P - pq - pk) / pph; pi = (P - pq - pk) % pph; }
  col = head * dh + hf * (dh / 2) + 16 * pi + jj;
}

__global__ __launch_bounds__(256) void pack_fp8_kernel(int mode, const bf16_t* s0, const bf16_t* s1,
                                                       const bf16_t* s2, int K, int N, int ld0,
                                                       int ld1, int ld2, int Hq, int Hkv, int dh,
                                                       const float* __restrict__ mul3,
                                                       const float* cm0, const float* cm1, const float* cm2,
                                                       uint4* __restrict__ dst) {
  const int kch = K / 128;
  const size_t total = static_cast<size_t>(N / 16) * kch * 2 * kWave;
  for (size_t g = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; g < total;
       g += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int lane = static_cast<int>(g % kWave);
    const int slot = static_cast<int>((g / kWave) % 2);
    const size_t fr = g / (2 * kWave);
    const int kf = static_cast<int>(fr % kch);
    const int nb = static_cast<int>(fr / kch);
    const int pc = 16 * nb + lane % 16;
    const int k0 = kf * 128 + 32 * (lane / 16) + 16 * slot;
    int col, which;
    packed_source(mode, pc, Hq, Hkv, dh, which, col);
    const bf16_t* src = which == 0 ? s0 : (which == 1 ? s1 : s2);
    const int ld = which == 0 ? ld0 : (which == 1 ? ld1 : ld2);
    const float* cm = which == 0 ? cm0 : (which == 1 ? cm1 : cm2);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = bf2f(src[static_cast<size_t>(k0 + i) * ld + col]);
    dst[g] = e4m3_pack16(v, cm ? cm[col] : mul3[which]);
  }
}

// Row-wise fp8 weights: per column of a [K][ld] bf16 tensor, one thread per
// column (consecutive threads, consecutive columns).
__global__ __launch_bounds__(256) void col_scales_kernel(const bf16_t* __restrict__ w, int K, int N, int ld,
                                                         float* __restrict__ mul, float* __restrict__ scale) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= N) return;
  float mx = 0.0f;
  for (int k = 0; k < K; ++k) mx = fmaxf(mx, fabsf(bf2f(w[static_cast<size_t>(k) * ld + j])));
  mul[j] = fp8_mul(mx);
  scale[j] = fp8_scale(mx);
}

__global__ __launch_bounds__(256) void pack_col_scales_kernel(int mode, const float* sc0, const float* sc1,
                                                              const float* sc2, int N, int Hq, int Hkv, int dh,
                                                              float* __restrict__ out) {
  const int pc = blockIdx.x * blockDim.x + threadIdx.x;
  if (pc >= N) return;
  int which, col;
  packed_source(mode, pc, Hq, Hkv, dh, which, col);
  out[pc] = (which == 0 ? sc0 : (which == 1 ? sc1 : sc2))[col];
}

// Row-wise codes of the adaRMS input: one 256-thread workgroup per row
// (float4 tid + 256 j of the row per thread, all in flight): r = 1 / rms,
// u = adaRMS(h) and max |u| over the row, then the row's codes (four per
// 32-bit word) from the same registers with its own scale.
__global__ __launch_bounds__(256) void rownorm_quant_kernel(const float* __restrict__ h, int D,
                                                            const float* __restrict__ scale,
                                                            const float* __restrict__ shift, float eps,
                                                            float* __restrict__ r_out, uint8_t* __restrict__ codes,
                                                            float* __restrict__ sx_row) {
  __shared__ float s_red[4];
  const int row = blockIdx.x, tid = threadIdx.x, n4 = D / 4;
  const float4* hr = reinterpret_cast<const float4*>(h + static_cast<size_t>(row) * D);
  float4 v[kNormPer];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int i = tid + 256 * j;
    v[j] = i < n4 ? hr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  ss = block_sum(ss, s_red);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  const float4* sc4 = reinterpret_cast<const float4*>(scale);
  const float4* sh4 = reinterpret_cast<const float4*>(shift);
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int i = tid + 256 * j;
    if (i >= n4) break;
    const float4 s = sc4[i], b = sh4[i];
    v[j] = make_float4(ada(v[j].x, r, s.x, b.x), ada(v[j].y, r, s.y, b.y), ada(v[j].z, r, s.z, b.z),
                       ada(v[j].w, r, s.w, b.w));
    mx = fmaxf(fmaxf(mx, fmaxf(fabsf(v[j].x), fabsf(v[j].y))), fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
  }
  mx = block_max(mx, s_red);
  const float mul = fp8_mul(mx);
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + static_cast<size_t>(row) * D);
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int i = tid + 256 * j;
    if (i >= n4) break;
    out[i] = e4m3_code(v[j].x * mul) | (e4m3_code(v[j].y * mul) << 8) | (e4m3_code(v[j].z * mul) << 16) |
             (e4m3_code(v[j].w * mul) << 24);
  }
  if (tid == 0) {
    r_out[row] = r;
    sx_row[row] = fp8_scale(mx);
  }
}

// Row-wise codes of bf16 rows (the attention output feeding an fp8 output
// projection): one 256-thread workgroup per row, eight values per uint4.
constexpr int kQbPer = 2;  // uint4 (8 values) per thread: K <= 256 * 8 * kQbPer

__global__ __launch_bounds__(256) void quant_bf16_rows_kernel(const bf16_t* __restrict__ src, int K,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ sx_row) {
  __shared__ float s_red[4];
  const int row = blockIdx.x, tid = threadIdx.x, n8 = K / 8;
  const uint4* sr = reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * K);
  float v[kQbPer][8];
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < kQbPer; ++j) {
    const int i = tid + 256 * j;
    const uint4 w = i < n8 ? sr[i] : make_uint4(0, 0, 0, 0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[j][2 * q] = __uint_as_float(ws[q] << 16);
      v[j][2 * q + 1] = __uint_as_float(ws[q] & 0xffff0000u);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) mx = fmaxf(mx, fabsf(v[j][q]));
  }
  mx = block_max(mx, s_red);
  const float mul = fp8_mul(mx);
  uint2* out = reinterpret_cast<uint2*>(codes + static_cast<size_t>(row) * K);
#pragma unroll
  for (int j = 0; j < kQbPer; ++j) {
    const int i = tid + 256 * j;
    if (i >= n8) break;
    uint32_t wd[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      wd[h2] = e4m3_code(v[j][4 * h2] * mul) | (e4m3_code(v[j][4 * h2 + 1] * mul) << 8) |
               (e4m3_code(v[j][4 * h2 + 2] * mul) << 16) | (e4m3_code(v[j][4 * h2 + 3] * mul) << 24);
    out[i] = make_uint2(wd[0], wd[1]);
  }
  if (tid == 0) sx_row[row] = fp8_scale(mx);
}

// bf16 weights in the same chunk order: [N/16][K/32][64 lanes][16 B] is
// already it (two consecutive k-fragments are one 64-wide chunk), so the
// bf16 GEMM reads the packing the other kernels use.

}  // namespace

hipError_t launch_rownorm(const float* h, int M, int D, const float* scale, const float* shift,
                          float eps, float* r, float* rowmax, hipStream_t s) {
  if (D % 4 || D > 4 * 256 * kNormPer) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rownorm_kernel, dim3(M), dim3(256), 0, s, h, M, D, scale, shift, eps, r, rowmax);
  return hipGetLastError();
}

hipError_t launch_quant(const float* src, const float* h, const float* r, const float* scale,
                        const float* shift, int M, int K, int T, const float* rowmax, int n_part,
                        int ldp, uint8_t* codes, float* sx_row, hipStream_t s) {
  if (K % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_kernel, dim3(M), dim3(256), 0, s, src, h, r, scale, shift, M, K, T, rowmax,
                     n_part, ldp, codes, sx_row);
  return hipGetLastError();
}

// The row tile: 32 rows.  At these row counts (at most a few hundred) the
// kernel is bound by load latency rather than operand reuse, so more and
// smaller tiles in flight win (800 x 1024 x 2048: 10 us with 32-row tiles,
// 16 us with 128-row tiles split over K).  K is split only when the tiles
// cover less than three quarters of the target.
TGemmPlan plan_tgemm(int M, int N, int K, int kc, int target_blocks) {
  TGemmPlan g;
  g.n_tiles = N / kBN;
  g.bm = 32;
  // very wide bf16 products (gate/up) have tiles to spare: 64-row tiles
  // there (800 x 8192 x 1024: 23.8 us against 26.3; the fp8 one is faster
  // with 32-row tiles, 20.7 against 24.8)
  if (kc == TOp<OP_BF16>::KC && ((M + 63) / 64) * g.n_tiles >= 3 * target_blocks) g.bm = 64;
  g.m_tiles = (M + g.bm - 1) / g.bm;
  const int chunks = K / kc;
  const int tiles = g.m_tiles * g.n_tiles;
  int s = 4 * tiles >= 3 * target_blocks ? 1 : (target_blocks + tiles - 1) / tiles;
  int max_s = chunks / 2 > 0 ? chunks / 2 : 1;  // at least two chunks per split
  if (max_s > kMaxSplit) max_s = kMaxSplit;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  g.ksplit = s;
  const int units = g.n_tiles * g.m_tiles * g.ksplit;
  g.blocks = kXcd * ((units + kXcd - 1) / kXcd);
  return g;
}

int tgemm_kc(int op) { return op == OP_FP8 ? TOp<OP_FP8>::KC : TOp<OP_BF16>::KC; }

size_t tgemm_partial_floats(const TGemmPlan& g) {
  return g.ksplit > 1 ? static_cast<size_t>(g.m_tiles) * g.n_tiles * g.ksplit * g.bm * kBN : 0;
}

// Two K chunks per LDS stage (half the barriers) pay off only on long K
// loops: down (64 chunks per tile) 21.5 -> 18.4 us, while 16-32 chunks lose
// 1-4 us (gate/up fp8 20.7 -> 24.4).
static bool two_chunk_stages(int n_chunks, int ksplit) {
  return n_chunks % 2 == 0 && n_chunks / ksplit >= 64;
}

hipError_t launch_tgemm(int op, Epilogue epi, const TGemmArgs& a0, int blocks, hipStream_t s) {
  if (a0.K % tgemm_kc(op) || a0.N % kBN) return hipErrorInvalidValue;
  TGemmArgs a = a0;
  a.main_blocks = blocks;
  dim3 grid(blocks + a.pf_blocks), block(kTT);
#define AE_TG(OPV, EPV, BMV)                                                                \
  if (op == OPV && epi == EPV && a.bm == BMV) {                                             \
    if (two_chunk_stages(a.K / tgemm_kc(op), a.ksplit))                                     \
      hipLaunchKernelGGL((tgemm_kernel<OPV, EPV, BMV, 2>), grid, block, 0, s, a);           \
    else                                                                                    \
      hipLaunchKernelGGL((tgemm_kernel<OPV, EPV, BMV, 1>), grid, block, 0, s, a);           \
    if (a.ksplit > 1) {                                                                     \
      const int tiles = a.n_tiles * a.m_tiles;                                              \
      if (a.M > 64 && tiles * ((a.M + 15) / 16) >= kRedSlicesWanted)                        \
        hipLaunchKernelGGL((tgemm_reduce_kernel<OPV, EPV, BMV, 16>), dim3(tiles * (BMV / 16)), \
                           block, 0, s, a);                                                 \
      else                                                                                  \
        hipLaunchKernelGGL((tgemm_reduce_kernel<OPV, EPV, BMV, 4>), dim3(tiles * (BMV / 4)),   \
                           block, 0, s, a);                                                 \
    }                                                                                       \
    return hipGetLastError();                                                               \
  }
#define AE_TG_BM(OPV, EPV) AE_TG(OPV, EPV, 64) AE_TG(OPV, EPV, 32)
  AE_TG_BM(OP_BF16, EPI_QKV)
  AE_TG_BM(OP_BF16, EPI_GELU)
  AE_TG_BM(OP_BF16, EPI_RESID)
  AE_TG_BM(OP_FP8, EPI_QKV)
  AE_TG_BM(OP_FP8, EPI_GELU)
  AE_TG_BM(OP_FP8, EPI_RESID)
#undef AE_TG_BM
#undef AE_TG
  return hipErrorInvalidValue;
}

hipError_t launch_weight_amax(const bf16_t* w, size_t n, unsigned* out, hipStream_t s) {
  hipLaunchKernelGGL(amax_kernel, dim3(512), dim3(256), 0, s, w, n, out);
  return hipGetLastError();
}

hipError_t launch_fp8_scales(const unsigned* amax_bits, int n, float* mul, float* scale,
                             hipStream_t s) {
  hipLaunchKernelGGL(scales_kernel, dim3((n + 63) / 64), dim3(64), 0, s, amax_bits, n, mul, scale);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(PackMode mode, const bf16_t* s0, const bf16_t* s1, const bf16_t* s2,
                           int K, int N, int ld0, int ld1, int ld2, int Hq, int Hkv, int dh,
                           const float* mul3, uint4* dst, hipStream_t s, const float* colmul0,
                           const float* colmul1, const float* colmul2) {
  if (K % 128 || N % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3(1024), dim3(256), 0, s, static_cast<int>(mode), s0, s1,
                     s2, K, N, ld0, ld1, ld2, Hq, Hkv, dh, mul3, colmul0, colmul1, colmul2, dst);
  return hipGetLastError();
}

hipError_t launch_fp8_col_scales(const bf16_t* w, int K, int N, int ld, float* mul, float* scale, hipStream_t s) {
  if (K < 1 || N < 1 || ld < N) return hipErrorInvalidValue;
  hipLaunchKernelGGL(col_scales_kernel, dim3((N + 255) / 256), dim3(256), 0, s, w, K, N, ld, mul, scale);
  return hipGetLastError();
}

hipError_t launch_pack_col_scales(PackMode mode, const float* sc0, const float* sc1, const float* sc2, int N,
                                  int Hq, int Hkv, int dh, float* out, hipStream_t s) {
  hipLaunchKernelGGL(pack_col_scales_kernel, dim3((N + 255) / 256), dim3(256), 0, s, static_cast<int>(mode), sc0,
                     sc1, sc2, N, Hq, Hkv, dh, out);
  return hipGetLastError();
}

hipError_t launch_rownorm_quant(const float* h, int M, int D, const float* scale, const float* shift, float eps,
                                float* r, uint8_t* codes, float* sx_row, hipStream_t s) {
  if (D % 4 || D > 4 * 256 * kNormPer) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rownorm_quant_kernel, dim3(M), dim3(256), 0, s, h, D, scale, shift, eps, r, codes, sx_row);
  return hipGetLastError();
}

hipError_t launch_quant_bf16_rows(const bf16_t* src, int M, int K, uint8_t* codes, float* sx_row, hipStream_t s) {
  if (K % 8 || K > 256 * 8 * kQbPer) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_bf16_rows_kernel, dim3(M), dim3(256), 0, s, src, K, codes, sx_row);
  return hipGetLastError();
}

}  // namespace ae
