// Host-side launch interface of the action-expert kernels (internal to the
// library; the public surface is include/ae.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ae {

enum Dt { DT_F32 = 0, DT_BF16 = 1 };

// Prologue of a projection GEMM: A is a bf16/fp32 activation matrix, or the
// fp32 residual h normalised on the fly by adaRMS.
enum Prologue { PRO_NONE = 0, PRO_ADARMS = 1 };
// Epilogue: RoPE + q / K-cache / V-cache scatter; gelu(gate) * up; gated
// residual update of h (+ row sums of squares for the next adaRMS).
enum Epilogue { EPI_QKV = 0, EPI_GELU = 1, EPI_RESID = 2 };
// Column order of a packed weight.
enum PackMode { PACK_PLAIN = 0, PACK_QKV = 1, PACK_GU = 2 };

constexpr int kMaxSteps = 64;  // Euler steps of one call at most
constexpr int kTileM = 64;  // rows per GEMM tile
constexpr int kTileN = 64;  // packed columns per GEMM tile (two 32-column pairs)

struct GemmArgs {
  // A operand
  const void* A;  // PRO_NONE: [M][lda] of the element type; PRO_ADARMS: fp32 h
  int lda;
  int M, K;
  // packed weight fragments and tiling
  const uint4* W;
  int n_tiles, m_tiles, k_frags, ksplit;
  // adaRMS
  const float* ssq;  // [ssq_tiles][ldssq] partial row sums of h^2
  int ssq_tiles, ldssq;
  const float* scale;
  const float* shift;
  float eps;
  // split-K scratch (zeroed counters, self-resetting)
  float* partial;
  int* counters;
  // EPI_RESID
  float* h;
  int ldh;
  const float* gate;
  float* ssq_out;
  // EPI_GELU
  void* out;
  int ldo;
  // EPI_QKV
  void* q;
  int ldq;
  void* kcache;   // layer's K cache, [Bmax][Hkv] x S_max keys x dh (key-block layout)
  void* vtcache;  // layer's V cache, same shape and layout family
  const int* n_valid;
  const float* rope_cos;  // [B][T][dh/2]
  const float* rope_sin;
  int T, Hq, Hkv, dh, S_max;
};

struct AttnArgs {
  const void* q;
  int ldq;
  const void* kcache;
  const void* vtcache;
  int S_max;
  const int* n_valid;
  void* o;
  int ldo;
  int T, Hq, Hkv, dh;
  // keys of request b: cache rows [0, n_valid[b] + n_act) (n_act = T: the
  // action tokens' own rows follow the prefix; 0: the prefix alone); a query
  // with no key gets zeros
  int n_act;
  int batch, n_qg, nsplit, kc_len;
  float scale_log2;
  float* partial;
  int* counters;
  // Extra workgroups past the attention's that read the weights the next
  // kernels multiply, so those arrive from the last-level cache instead of
  // HBM (pf_blocks == 0: none).  Ranges of 16-byte words.
  const uint4* pf[4];
  int pf_n4[4];
  int pf_blocks;
};

// Split-K / grid planning shared by the runtime and the launchers.
struct GemmPlan {
  int m_tiles, n_tiles, k_frags, ksplit, blocks;
};
GemmPlan plan_gemm(Dt dt, int M, int N, int K, int target_blocks);
int kstep_of(Dt dt);

hipError_t launch_gemm(Dt dt, Prologue pro, Epilogue epi, const GemmArgs& a, int blocks,
                       hipStream_t s);
hipError_t launch_attention(Dt dt, const AttnArgs& a, hipStream_t s);
// partial scratch of a key-split launch; rows_per_item query rows per item
size_t attention_partial_floats(int dh, int items, int nsplit, int rows_per_item);
// query rows one item of the batched attention kernel covers
int attention_rows_per_item();
// key splits the batched attention kernel uses at most for `items` items
int attention_max_splits(int items);

hipError_t launch_tpath_sinusoid(float* e, int n_steps, int width, hipStream_t s);
// p[0 .. n) = 0 with a kernel (a fill a captured graph can hold)
hipError_t launch_zero_ints(int* p, size_t n, hipStream_t s);
// out[k][l][n] = sum_d mod[k][l][which][d] * W_l[d][n] for packed weights
// (n in packed column order), steps k < n_steps, layers l < L, with nchunk
// modulation chunks of D per layer (6 joint, 9 DiT-style).
hipError_t launch_shift_bias(Dt dt, const uint4* W, size_t layer_stride, int K, int N, const float* mod,
                             int n_steps, int L, int D, int nchunk, int which, float* out, hipStream_t s);
// Y[m][n] = act(sum_k X[m][k] W[k][n] + b[n]), m < M <= 16; act 0 none, 1 SiLU.
// grid.y = n_mat matrices with strides (W, b, Y advance by the given strides).
hipError_t launch_gemv_rows(Dt dt, const float* X, int ldx, int M, int K, const void* W, int ldw,
                            const void* b, int N, float* Y, int ldy, int act, int n_mat,
                            size_t w_stride, size_t b_stride, size_t y_stride, hipStream_t s);

// (ha, sc optional: ha = bf16(h (1 + sc)) for a norm applied after the
// next product)
hipError_t launch_action_in(const float* x, int M, int A, const float* w_in, const float* b_in,
                            float* h, int D, float* ssq, int ldssq, hipStream_t s,
                            uint16_t* ha = nullptr, const float* sc = nullptr);
hipError_t launch_action_out(float* x, int M, int A, const float* h, int D, const float* scale,
                             const float* shift, float eps, const float* w_out,
                             const float* b_out, float dt, hipStream_t s);

// (extra: visible rows that follow the P mask rows, e.g. the robot state's:
// they count into n_valid; src_of, when set: its inverse, src_of[b P + key]
// = the row holding visible key `key`)
hipError_t launch_prefix_scan(const uint8_t* mask, int batch, int P, int* comp_idx, int* n_valid,
                              int T, int dh, float theta, float* rope_cos, float* rope_sin,
                              hipStream_t s, int extra = 0, int* src_of = nullptr);
// cos / sin of RoPE at positions 0 .. n_pos - 1: [n_pos][dh / 2] fp32 (double math)
hipError_t launch_pos_table(int n_pos, int dh, float theta, float* cos_t, float* sin_t, hipStream_t s);
// The robot state's context row: out[b] = bf16(state[b] . W + bias) ([S] x [S][D]
// bf16 + [D] bf16), and its key, key_out[b] = n_valid[b] - 1 (the last visible row).
hipError_t launch_state_prep(const float* state, int batch, int S, const uint16_t* w, const uint16_t* bias,
                             int D, const int* n_valid, uint16_t* out, int* key_out, hipStream_t s);
// K / V [L][batch][P][Hkv][dh] visible rows -> keys 0 .. n_valid[b] - 1 of
// the key-block caches (src_of from launch_prefix_scan); K null: only the
// finite fill past n_valid + n_act
hipError_t launch_prefix_copy(Dt dt, const void* K, const void* V, const int* src_of,
                              const int* n_valid, int n_act, int L, int batch, int P, int Hkv, int dh,
                              int Bmax, int S_max, void* kcache, void* vtcache, hipStream_t s);

// Pack logical [K][N] row-major sources into MFMA fragment order; rows
// k >= kvalid and columns n >= nvalid (PACK_PLAIN) read as zero (padding).
hipError_t launch_pack(Dt dt, PackMode mode, const void* s0, const void* s1, const void* s2,
                       int K, int N, int ld0, int ld1, int ld2, int Hq, int Hkv, int dh,
                       uint4* dst, hipStream_t s, int kvalid = -1, int nvalid = -1);
// fp32 copy of src (n elements); transpose_cols > 0 also transposes a
// [n / transpose_cols][transpose_cols] matrix.
hipError_t launch_to_f32(Dt dt, const void* src, float* dst, size_t n, int transpose_cols,
                         hipStream_t s);

// ---------------------------------------------------------------------------
// Batched tiled GEMM (128 x 128 tiles through LDS) with bf16 or fp8 e4m3
// operands, and the row-norm / quantise passes in front of it.
// ---------------------------------------------------------------------------

enum Operand { OP_BF16 = 0, OP_FP8 = 1 };

struct TGemmArgs {
  const void* A;  // [M][lda] operand-typed rows (bf16 or e4m3 codes)
  size_t lda_bytes;
  int M, N, K;
  const uint4* W;  // packed weights (bf16 fragments or fp8 chunks)
  int n_tiles, m_tiles, ksplit;
  int bm;  // tile rows (32 or 64)
  // optional prefetch workgroups past the tile grid (as in AttnArgs): they
  // read pf ranges into the last-level cache; main_blocks is set by
  // launch_tgemm
  const uint4* pf[2];
  int pf_n4[2];
  int pf_blocks, main_blocks;
  float* partial;
  int* counters;
  // fp8: per-row activation scale and per-tensor weight scales, or (swc
  // set: row-wise scaling) one weight scale per packed output column
  const float* sx_row;
  const float* sw;
  const float* swc;
  // EPI_RESID
  float* h;
  int ldh;
  const float* gate;
  // EPI_GELU (fp8: fp32 out plus per-(n-tile, row) max |out|)
  void* out;
  int ldo;
  float* rowmax;
  int ldp;
  // EPI_QKV
  void* q;
  int ldq;
  void* kcache;
  void* vtcache;
  const int* n_valid;
  const float* rope_cos;
  const float* rope_sin;
  int T, Hq, Hkv, dh, S_max;
  // EPI_QKV on context rows (key_map set): row m of request m / T goes to
  // cache key key_map[m] (< 0: not stored), its K rotated at that position
  // with pos_cos / pos_sin [position][dh / 2]
  const int* key_map;
  const float* pos_cos;
  const float* pos_sin;
  // several layers' context products in one launch: columns [l c, (l + 1) c)
  // with c = ctx_layer_cols belong to layer l, whose A rows start
  // a_layer_bytes past layer 0's (0: every layer multiplies the same rows,
  // as the state rows do) and whose caches start ctx_layer_elems elements
  // past layer 0's (ctx_layer_cols 0: one layer)
  int ctx_layer_cols;
  size_t ctx_layer_elems;
  size_t a_layer_bytes;
  // bf16 norm after the product (A = bf16(h (1 + scale))): EPI_QKV / EPI_GELU
  // finish with y = r_row acc + bias[col], r_row from the row sums of squares
  // ssq[ssq_tiles][ldssq] (64-column partials over K columns); EPI_RESID
  // writes those partials of the new h and, when nsc is set, the next norm's
  // ha = bf16(h (1 + nsc))
  const float* bias;
  float* ssq;
  int ldssq, ssq_tiles;
  float eps;
  const float* nsc;
  uint16_t* ha;
};

struct TGemmPlan {
  int m_tiles, n_tiles, ksplit, blocks;
  int bm;  // tile rows
};
TGemmPlan plan_tgemm(int M, int N, int K, int kc, int target_blocks);
int tgemm_kc(int op);
size_t tgemm_partial_floats(const TGemmPlan& g);
hipError_t launch_tgemm(int op, Epilogue epi, const TGemmArgs& a, int blocks, hipStream_t s);

// per-row r = 1 / rms(h) and max |adaRMS(h)| (the fp8 inputs' norm)
hipError_t launch_rownorm(const float* h, int M, int D, const float* scale, const float* shift,
                          float eps, float* r, float* rowmax, hipStream_t s);
// e4m3 codes of fp32 rows (src) or of u recomputed from h and r (src null),
// scaled per request by the amax over rowmax[n_part][ldp] of its rows
hipError_t launch_quant(const float* src, const float* h, const float* r, const float* scale,
                        const float* shift, int M, int K, int T, const float* rowmax, int n_part,
                        int ldp, uint8_t* codes, float* sx_row, hipStream_t s);
// fp8 weights: per-tensor amax (atomic max of the bit patterns into a zeroed
// word), the (448 / amax, amax / 448) pairs, and the packed codes
hipError_t launch_weight_amax(const uint16_t* w, size_t n, unsigned* out, hipStream_t s);
hipError_t launch_fp8_scales(const unsigned* amax_bits, int n, float* mul, float* scale,
                             hipStream_t s);
// Row-wise fp8: per output column of a bf16 weight [K][ld] (first N
// columns) the multiplier 448 / amax and the scale amax / 448 (amax floored
// at 1e-12), both fp32.
hipError_t launch_fp8_col_scales(const uint16_t* w, int K, int N, int ld, float* mul, float* scale, hipStream_t s);
// The scale of every packed column: out[pc] = scale of the logical column
// packed at pc (the packing's column map; sc1 / sc2 unused by PACK_PLAIN).
hipError_t launch_pack_col_scales(PackMode mode, const float* sc0, const float* sc1, const float* sc2, int N,
                                  int Hq, int Hkv, int dh, float* out, hipStream_t s);
// Row-wise fp8 activations: one workgroup per row.  norm: r = 1 / rms(h),
// u = adaRMS(h), codes of u with the row's own scale (D <= 4096); bf16 rows:
// codes of the row as it is (K <= 4096).
hipError_t launch_rownorm_quant(const float* h, int M, int D, const float* scale, const float* shift, float eps,
                                float* r, uint8_t* codes, float* sx_row, hipStream_t s);
hipError_t launch_quant_bf16_rows(const uint16_t* src, int M, int K, uint8_t* codes, float* sx_row,
                                  hipStream_t s);
// Packs fp8 weights; colmul (per source: its per-column multipliers, or all
// null: mul3 per source) sets the row-wise scaling.
hipError_t launch_pack_fp8(PackMode mode, const uint16_t* s0, const uint16_t* s1, const uint16_t* s2,
                           int K, int N, int ld0, int ld1, int ld2, int Hq, int Hkv, int dh,
                           const float* mul3, uint4* dst, hipStream_t s, const float* colmul0 = nullptr,
                           const float* colmul1 = nullptr, const float* colmul2 = nullptr);

// ---------------------------------------------------------------------------
// Persistent whole-call kernel (batch * T <= 64 rows)
// ---------------------------------------------------------------------------

struct PGemm {
  int n_tiles, k_frags, ksplit;
  int nb;  // 16-column groups per tile: 4 (64 columns) or 2 (32 columns, bf16)
};

struct PersistArgs {
  int M, D, L, n_steps, T, A, Hq, Hkv, dh, F, S_max, qdim, ssq_tiles, ldssq, batch, G;
  float eps, dt, scale_log2;
  const uint4 *wqkv, *wo, *wgu, *wd;
  size_t sqkv, so, sgu, sd;
  const uint4* win_p;   // W_in packed: K = A (padded), N = D
  const uint4* wout_p;  // W_out packed: K = D, N = A (padded to 16s)
  int a_frags, a_blocks;
  const float *b_in, *b_out;
  const float *mod, *fmod;
  void *kcache, *vtcache;
  size_t kv_layer;  // elements per layer of each cache
  const int* n_valid;
  const float *rope_cos, *rope_sin;
  float *x, *h, *ssq;
  void *q, *o, *act;
  void* ha;              // T [M][D]: h (1 + scale) of the norm that reads h next
  const float *bq, *bg;  // [steps][L][N]: shift W of the QKV and gate/up norms
  int qkv_n;
  float* gpart;  // split-K partials as (value, generation) packets
  int* gcnt;
  float* apart;
  int* acnt;   // attention split counters (= pcnt + GEMM tile counters)
  int* pcnt;   // monotonic split counters: q, o, gate/up, down tiles, then attention items
  int n_acnt;  // attention items
  int* flags;  // [G] barrier generations
  uint32_t* genp;  // [2] split-K packet generation base: next launch's, this launch's
  int* err;    // [2]: this launch's error flag (a wait timed out), launches that raised it
  PGemm pq, po, pg, pd;
  int n_qg, nsplit, kc_len;
};

int persist_kpw();
int persist_max_grid();
int persist_blocks_per_cu(Dt dt, int dh);
hipError_t launch_persist(Dt dt, const PersistArgs& a, hipStream_t s);

}  // namespace ae
