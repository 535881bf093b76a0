// Host runtime behind include/ae.h: config validation, the static buffer
// plan (every device buffer is allocated in ae_create, none lazily), weight
// ingest and packing, prefix ingest, step sequencing and hipGraph capture /
// replay of whole denoise calls keyed by (batch, steps, prefix bucket).
//
// The library follows the MolmoBot PR (Part 1: graph inputs are static
// buffers allocated up front, never lazily built; Part 2: the context K/V is
// ingested once per query and every step reads it) and the sglang PR summary
// (item 3: a bounded LRU graph cache whose evicted graphs are released, or
// direct launches when it is full; item 4: prefix buckets, and the mutable
// prefix K/V and mask refreshed in place before a replay; item 5: bucket
// lengths validated up front).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/ae.h"
#include "ae_graph_cache.h"
#include "ae_kernels.h"

using namespace ae;

namespace {

constexpr int kTargetBlocks = 256;  // one workgroup per CU at least
constexpr int kPrefetchBlocks = 32;  // weight-prefetch workgroups beside the batched attention
constexpr int kMaxGraphs = 64;   // graph_cache_size at most
constexpr int kMaxBuckets = 32;  // prefix bucket lengths at most
// Key splits per attention item in the whole-call kernel at most: past ~16
// the distributed merge costs more than the shorter key loop saves (the
// MolmoBot-shaped expert, 4 items over 2064 keys: 33 splits 6.73 ms per call,
// 16 splits 6.38, 8 splits 6.43; the Pi0.5 shape plans 12 either way).
constexpr int kPersistMaxSplits = 16;

// A cached graph and an event recorded after its latest replay: an evicted
// graph is destroyed only once that event has completed.
struct GraphEntry {
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;
  size_t nodes = 0;  // of the captured graph
};


struct Buf {
  void* p = nullptr;
  size_t bytes = 0;
};

// The transient device memory a denoise call's kernels work in: split-K
// partials and counters, attention key-split partials and counters, and the
// whole-call kernel's barrier flags, split counters and packet generation
// base.  A handle owns one set sized for its largest call.
struct ScratchSet {
  float* gpart = nullptr;   // split-K partials ((value, generation) packets in the whole-call kernel)
  int* gcnt = nullptr;      // per-tile split counters (self-resetting)
  float* apart = nullptr;   // attention key-split partials
  int* acnt = nullptr;      // per-item split counters (self-resetting)
  int* flags = nullptr;     // whole-call kernel: barrier generation per workgroup
  int* pcnt = nullptr;      // whole-call kernel: monotonic split counters
  uint32_t* genp = nullptr; // whole-call kernel: [2] next / current packet generation base
};

// Element counts of a scratch set's parts.
struct ScratchNeed {
  size_t gfl = 0, gcn = 0, afl = 0, acn = 0, flags = 1, pcnt = 1;
  void max_with(const ScratchNeed& o) {
    gfl = std::max(gfl, o.gfl); gcn = std::max(gcn, o.gcn); afl = std::max(afl, o.afl);
    acn = std::max(acn, o.acn); flags = std::max(flags, o.flags); pcnt = std::max(pcnt, o.pcnt);
  }
};

}  // namespace

struct ae_handle {
  ae_config cfg{};
  Dt dt = DT_BF16;
  int esz = 2;
  int L = 0, D = 0, Hq = 0, Hkv = 0, dh = 0, F = 0, T = 0, A = 0, Pmax = 0, Bmax = 0, Nmax = 0;
  int S_max = 0, qdim = 0, kvdim = 0, qkv_n = 0, ssq_tiles = 0, Mmax = 0;
  int Dc = 0, Sd = 0;  // context width and robot-state size (0: no context preparation)
  bool dit = false;    // DiT-style block: attn1 over the action tokens, attn2 over the prefix
  int nmod = 6;        // modulation chunks of D per layer (9 in the DiT-style block)

  // weights (library-owned copies)
  void *tw1 = nullptr, *tb1 = nullptr, *tw2 = nullptr, *tb2 = nullptr;
  void *fmod_w = nullptr, *fmod_b = nullptr, *mod_w = nullptr, *mod_b = nullptr;
  float *w_in = nullptr, *b_in = nullptr, *w_out = nullptr, *b_out = nullptr;
  uint4 *wqkv = nullptr, *wo = nullptr, *wgu = nullptr, *wd = nullptr;
  size_t sqkv = 0, so = 0, sgu = 0, sd = 0;  // per-layer strides in uint4
  // DiT-style block: attn2's query and output projections (strides sq2, so)
  uint4 *wq2 = nullptr, *wo2 = nullptr;
  size_t sq2 = 0;

  // context preparation: each layer's [ctx_k | ctx_v] packed (RoPE pairs
  // together), RoPE tables of positions 0 .. max_prefix_len, the state's
  // input layer, its context row and cache key per request
  uint4* wctx = nullptr;
  size_t sctx = 0;  // per-layer stride in uint4
  float *pos_cos = nullptr, *pos_sin = nullptr;
  uint16_t *st_w = nullptr, *st_b = nullptr, *st_h = nullptr;
  int* st_key = nullptr;

  // prefix state
  void *kcache = nullptr, *vtcache = nullptr;
  // DiT-style block: attn1's K/V of the action rows alone ([L][Bmax][Hkv]
  // [S_self][dh]), read with the all-zero visible counts `zeros`
  void *kself = nullptr, *vtself = nullptr;
  int S_self = 0;
  int* zeros = nullptr;
  int *comp_idx = nullptr, *n_valid = nullptr;
  int* src_of = nullptr;  // inverse of comp_idx: the row of each visible key
  float *rope_cos = nullptr, *rope_sin = nullptr;

  // activations
  float *x = nullptr, *h = nullptr, *e = nullptr, *z = nullptr, *c = nullptr;
  float *mod = nullptr, *fmod = nullptr, *ssq = nullptr;
  void *q = nullptr, *o = nullptr, *act = nullptr;
  // whole-call kernel: the modulated shadow of h, and the norms' shift terms
  // folded through W_qkv / W_gate-up ([steps][L][N], packed column order)
  void* ha = nullptr;
  float *bq = nullptr, *bg = nullptr;
  float* bq2 = nullptr;  // DiT-style block: attn2's shift through W_q2 ([steps][L][qdim])

  // split scratch of this handle's calls
  ScratchSet own;

  // batched tiled path: bf16, or fp8 e4m3 QKV / gate-up / down projections
  bool tiled = false;
  bool fp8 = false;
  bool rowwise = false;  // fp8 scales per weight column and per activation row
  bool fp8o = false;     // fp8 attention output projection (row-wise)
  // row-wise: each layer's weight scales per packed column of qkv, gate-up,
  // down and (fp8o) o, at offsets 0, qkv_n, qkv_n + 2F, qkv_n + 2F + D
  float* swc = nullptr;
  size_t swc_layer = 0;
  float *cmul = nullptr, *csc = nullptr;  // per logical column of one layer's tensors (weight load)
  void* ubuf = nullptr;  // fp8 GEMM input rows (e4m3 codes)
  float *rrow = nullptr, *rowmax = nullptr, *sxrow = nullptr;
  unsigned* wamax = nullptr;             // [L][6] amax bits of q, k, v, gate, up, down
  float *wmul = nullptr, *wsc = nullptr;  // [L][6] 448 / amax and amax / 448

  // persistent whole-call kernel (batch * T <= 64)
  uint4 *win_p = nullptr, *wout_p = nullptr;
  int a_frags = 0, a_blocks = 0;
  int* derr = nullptr;  // [2] the whole-call kernel's error flag and count
  int G = 0;              // resident workgroups of the persistent kernel (0: unavailable)
  int device = 0;         // the device the handle was created on
  bool persist_graph = true;  // cooperative launch can be captured

  bool weights_loaded = false;
  int prefix_batch = -1;
  int table_steps = -1;  // step count the modulation table currently holds
  hipStream_t cap_stream = nullptr;
  LruCache<CallKey, GraphEntry> graphs;
  std::vector<GraphEntry> retired;  // evicted, destroyed once their last replay is done
  std::vector<int> buckets;         // prefix bucket lengths (ascending); empty: one bucket
  int span = 0;                     // key span of the current prefix: its bucket length
  ae_stats stats{};
  std::string err;
  std::vector<Buf> bufs;
};

namespace {

ae_status fail(ae_handle* h, ae_status s, const std::string& msg) {
  if (h) h->err = msg;
  return s;
}

ae_status hip_fail(ae_handle* h, hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return fail(h, AE_ERR_HIP, m);
}

#define AE_HIP(h, call)                                   \
  do {                                                    \
    hipError_t e_ = (call);                               \
    if (e_ != hipSuccess) return hip_fail((h), e_, #call); \
  } while (0)

template <typename P>
ae_status alloc(ae_handle* h, P** out, size_t bytes) {
  void* p = nullptr;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, AE_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
  }
  h->bufs.push_back({p, bytes});
  h->stats.device_bytes += static_cast<long long>(bytes);
  *out = static_cast<P*>(p);
  return AE_OK;
}

std::string validate_config(const ae_config* c) {
  if (c->n_layers < 1) return "n_layers must be >= 1";
  if (c->width < 64 || c->width % 64) return "width must be a positive multiple of 64";
  if (c->width > 4096) return "width above 4096 is not supported";
  if (c->n_q_heads < 1 || c->n_kv_heads < 1) return "head counts must be >= 1";
  if (c->n_q_heads % c->n_kv_heads) return "n_kv_heads must divide n_q_heads";
  if (c->mlp_dim < 32 || c->mlp_dim % 32) return "mlp_dim must be a positive multiple of 32";
  if (c->action_horizon < 1) return "action_horizon must be >= 1";
  if (c->action_dim < 1 || c->action_dim > 64) return "action_dim must be in [1, 64]";
  if (c->max_prefix_len < 0) return "max_prefix_len must be >= 0";
  if (c->max_batch < 1) return "max_batch must be >= 1";
  if (c->max_steps < 1 || c->max_steps > kMaxSteps) return "max_steps must be in [1, 64]";
  if (c->act_dtype != AE_F32 && c->act_dtype != AE_BF16) return "act_dtype must be AE_F32 or AE_BF16";
  if (!(c->rope_theta > 0.0f)) return "rope_theta must be > 0";
  if (!(c->rms_eps >= 0.0f)) return "rms_eps must be >= 0";
  if (c->use_graphs != 0 && c->use_graphs != 1) return "use_graphs must be 0 or 1";
  if (c->graph_cache_size < 0 || c->graph_cache_size > kMaxGraphs) return "graph_cache_size must be in [0, 64]";
  if (c->graph_cache_evict != 0 && c->graph_cache_evict != 1) return "graph_cache_evict must be 0 or 1";
  if (c->context_width < 0 || c->context_width % 64 || c->context_width > 8192)
    return "context_width must be 0 or a multiple of 64 up to 8192";
  if (c->state_dim < 0 || c->state_dim > 64) return "state_dim must be in [0, 64]";
  if (c->state_dim > 0 && c->context_width == 0) return "state_dim needs context_width";
  if (c->block_type != AE_BLOCK_JOINT && c->block_type != AE_BLOCK_DIT)
    return "block_type must be AE_BLOCK_JOINT or AE_BLOCK_DIT";
  if ((c->fp8_rowwise != 0 && c->fp8_rowwise != 1) || (c->fp8_oproj != 0 && c->fp8_oproj != 1))
    return "fp8_rowwise and fp8_oproj must be 0 or 1";
  if ((c->fp8_rowwise || c->fp8_oproj) && c->proj_weight_dtype != AE_FP8_E4M3)
    return "fp8_rowwise / fp8_oproj need proj_weight_dtype AE_FP8_E4M3";
  if (c->exec_path < AE_PATH_AUTO || c->exec_path > AE_PATH_PER_PHASE)
    return "exec_path must be AE_PATH_AUTO, AE_PATH_WHOLE_CALL or AE_PATH_PER_PHASE";
  return "";
}

std::string unsupported_config(const ae_config* c) {
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return "head_dim must be 64, 128 or 256";
  if (c->context_width > 0 && (c->act_dtype != AE_BF16 || (2 * c->n_kv_heads * c->head_dim) % 128))
    return "context preparation needs bf16 and 2 n_kv_heads head_dim a multiple of 128";
  if (c->fp8_oproj && (!c->fp8_rowwise || (c->n_q_heads * c->head_dim) % 128))
    return "fp8_oproj needs fp8_rowwise and n_q_heads * head_dim a multiple of 128";
  if (c->block_type == AE_BLOCK_DIT) {
    const int qd = c->n_q_heads * c->head_dim, qkv = qd + 2 * c->n_kv_heads * c->head_dim;
    if (c->act_dtype != AE_BF16 || c->proj_weight_dtype != AE_BF16)
      return "the DiT-style block needs bf16 weights and projections";
    if (c->width % 128 || qkv % 128 || qd % 128 || (2 * c->mlp_dim) % 128 || c->mlp_dim % 64)
      return "the DiT-style block needs width, n_q_heads head_dim, (n_q_heads + 2 n_kv_heads) "
             "head_dim and 2 mlp_dim to be multiples of 128";
  }
  if (c->proj_weight_dtype != c->act_dtype) {
    if (c->proj_weight_dtype != AE_FP8_E4M3 || c->act_dtype != AE_BF16)
      return "proj_weight_dtype must equal act_dtype (or be AE_FP8_E4M3 with bf16)";
    const int qkv_n = (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
    if (c->width % 128 || c->mlp_dim % 128 || qkv_n % 128)
      return "fp8 projections need width, mlp_dim and (n_q_heads + 2 n_kv_heads) * head_dim "
             "to be multiples of 128";
  }
  return "";
}

size_t elems_packed(int K, int N, int kstep) {
  // [N/16][K/kstep][64 lanes] x 16 bytes, in uint4 units
  return static_cast<size_t>(N / 16) * (K / kstep) * 64;
}

struct AttnPlan {
  int n_qg, nsplit, kc_len, items;
};

// rows: query rows one item covers (64 in the whole-call kernel, the batched
// kernel's attention_rows_per_item() otherwise)
// span: the prefix bucket (visible rows at most)
AttnPlan plan_attention(const ae_handle* h, int batch, int span, int rows, int max_splits = 1 << 30) {
  AttnPlan a;
  const int R = h->T * (h->Hq / h->Hkv);
  a.n_qg = (R + rows - 1) / rows;
  a.items = batch * h->Hkv * a.n_qg;
  const int kstep = kstep_of(h->dt);
  const int max_keys = span + h->T;
  int ns = (kTargetBlocks + a.items - 1) / a.items;
  const int max_ns = (max_keys + 63) / 64;
  if (ns > max_ns) ns = max_ns;
  if (ns > max_splits) ns = max_splits;
  if (ns < 1) ns = 1;
  int kc = (max_keys + ns - 1) / ns;
  kc = (kc + kstep - 1) / kstep * kstep;
  a.kc_len = kc;
  a.nsplit = (max_keys + kc - 1) / kc;
  return a;
}

// The batched attention kernel's plan.
AttnPlan plan_attention_batched(const ae_handle* h, int batch, int span) {
  const int rows = attention_rows_per_item();
  const int R = h->T * (h->Hq / h->Hkv);
  const int items = batch * h->Hkv * ((R + rows - 1) / rows);
  return plan_attention(h, batch, span, rows, attention_max_splits(items));
}

// Largest key split count a plan can choose for `items` items at any span
// up to the capacity (sizes the partial scratch for every bucket).
int max_attention_splits(const ae_handle* h, int items, int max_splits) {
  int ns = (kTargetBlocks + items - 1) / items;
  ns = std::min(ns, (h->Pmax + h->T + 63) / 64);
  ns = std::min(ns, max_splits);
  return std::max(ns, 1);
}

// The projection GEMMs of one layer: qkv, o, gate/up, down.
struct LayerPlans {
  GemmPlan qkv, o, gu, d;
};

LayerPlans plan_layer(const ae_handle* h, int M) {
  LayerPlans p;
  p.qkv = plan_gemm(h->dt, M, h->qkv_n, h->D, kTargetBlocks);
  p.o = plan_gemm(h->dt, M, h->D, h->qdim, kTargetBlocks);
  p.gu = plan_gemm(h->dt, M, 2 * h->F, h->D, kTargetBlocks);
  p.d = plan_gemm(h->dt, M, h->D, h->F, kTargetBlocks);
  return p;
}

// Persistent path: one row tile; split K so that the tasks of a phase cover
// the resident workgroups once and every wave holds at most persist_kpw()
// weight fragments in registers.
PGemm plan_pgemm(const ae_handle* h, int N, int K) {
  PGemm g;
  g.nb = kTileN / 16;
  g.n_tiles = N / kTileN;
  g.k_frags = K / kstep_of(h->dt);
  int s = h->G / g.n_tiles;
  const int kpw = persist_kpw();
  const int min_s = (g.k_frags + 4 * kpw - 1) / (4 * kpw);
  if (s < min_s) s = min_s;
  if (s > g.k_frags) s = g.k_frags;
  if (s < 1) s = 1;
  g.ksplit = s;
  return g;
}

struct PersistPlans {
  PGemm q, o, g, d;
};

// The same product in 32-column tiles with the whole K range per task (bf16,
// K / 32 <= 8 fragments per wave): no split, so no exchange of partials
// between workgroups, but each task reads all of A (twice the A bytes per
// workgroup).  Taken only where these tasks alone cover every workgroup;
// with fewer the idle CUs cost more than the exchange saves.  Measured on
// the Pi0.5 shape: gate/up (256 tasks) 11.80 -> 11.63 ms per call; QKV (80
// tasks) 12.17, both 11.94; on the MolmoBot shape gate/up (192 tasks) 6.61
// -> 6.73.  Returns false where it does not apply.
bool plan_pgemm_narrow(const ae_handle* h, int N, int K, PGemm& g) {
  if (h->dt != DT_BF16 || N % 32 || K % 32) return false;
  const int kf = K / kstep_of(h->dt);
  if (kf > 4 * 2 * persist_kpw() || N / 32 < h->G) return false;
  g.nb = 2;
  g.n_tiles = N / 32;
  g.k_frags = kf;
  g.ksplit = 1;
  return true;
}

// K splits of the QKV phase at most: its reducers also rotate and scatter
// q / K / V, and fewer, longer members measured faster there (Pi0.5 shape:
// 6 splits 12.2 ms per call, 4 splits 11.75, 2 splits 11.8, 8 splits 13.3;
// the MolmoBot shape goes from 12 to 4 at +0.1 ms); the other phases keep
// the plan that covers the workgroups (fewer splits there measured slower).
constexpr int kPersistQkvMaxSplits = 4;

PersistPlans plan_persist(const ae_handle* h) {
  PersistPlans p;
  p.q = plan_pgemm(h, h->qkv_n, h->D);
  {
    const int min_s = (p.q.k_frags + 4 * persist_kpw() - 1) / (4 * persist_kpw());
    p.q.ksplit = std::max(min_s, std::min(p.q.ksplit, kPersistQkvMaxSplits));
  }
  p.o = plan_pgemm(h, h->D, h->qdim);
  p.g = plan_pgemm(h, 2 * h->F, h->D);
  p.d = plan_pgemm(h, h->D, h->F);
  PGemm n;  // (QKV keeps its split: 80 narrow tasks measured slower)
  if (plan_pgemm_narrow(h, 2 * h->F, h->D, n)) p.g = n;
  return p;
}

// The whole-call kernel covers one 64-row tile and action_dim <= 32; other
// shapes run the per-phase kernels.  Of the calls it covers, AE_PATH_AUTO
// gives it those whose layer weights exceed the last-level cache: below
// that the per-phase kernels find a step's weights still cached from the
// previous step and win (the MolmoBot-shaped expert, 208 MB of weights, by
// ~15 % at batch 1 and more at batch 4; the Pi0.5 shape cut to 6 layers,
// 207 MB, by ~5 %), while above it the whole-call kernel wins (the Pi0.5
// shape, 623 MB, by ~2-4 %): its time per layer is its synchronisation
// chain whether the weights are cached or not.
constexpr size_t kLastLevelCacheBytes = static_cast<size_t>(256) << 20;

size_t layer_weight_bytes(const ae_handle* h) {
  return static_cast<size_t>(h->L) * (h->sqkv + h->so + h->sgu + h->sd) * 16;
}

bool use_persist(const ae_handle* h, int batch) {
  if (!(h->G > 0 && !h->fp8 && !h->dit && batch * h->T <= kTileM && h->A <= 32)) return false;
  if (h->cfg.exec_path == AE_PATH_WHOLE_CALL) return true;
  if (h->cfg.exec_path == AE_PATH_PER_PHASE) return false;
  return layer_weight_bytes(h) > kLastLevelCacheBytes;
}

// The batched tiled path: the four projection GEMMs of a layer.
struct TPlans {
  int op;
  TGemmPlan qkv, o, gu, d;
  TGemmPlan q2;  // DiT-style block: attn2's queries
};

TPlans plan_tlayer(const ae_handle* h, int M) {
  TPlans p;
  p.op = h->fp8 ? OP_FP8 : OP_BF16;
  const int kc = tgemm_kc(p.op), kb = tgemm_kc(OP_BF16);
  p.qkv = plan_tgemm(M, h->qkv_n, h->D, kc, kTargetBlocks);
  p.o = plan_tgemm(M, h->D, h->qdim, h->fp8o ? kc : kb, kTargetBlocks);
  p.gu = plan_tgemm(M, 2 * h->F, h->D, kc, kTargetBlocks);
  p.d = plan_tgemm(M, h->D, h->F, kc, kTargetBlocks);
  p.q2 = plan_tgemm(M, h->qdim, h->D, kb, kTargetBlocks);
  return p;
}

TGemmArgs base_tgemm(const ae_handle* h, const ScratchSet& sc, const TGemmPlan& g, int M, int N, int K) {
  TGemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = M; a.N = N; a.K = K;
  a.n_tiles = g.n_tiles; a.m_tiles = g.m_tiles; a.ksplit = g.ksplit; a.bm = g.bm;
  a.partial = sc.gpart; a.counters = sc.gcnt;
  a.sx_row = h->sxrow;
  return a;
}

size_t gemm_scratch_floats(const GemmPlan& g) {
  return g.ksplit > 1 ? static_cast<size_t>(g.m_tiles) * g.n_tiles * g.ksplit * kTileM * kTileN : 0;
}

GemmArgs base_gemm(const ae_handle* h, const ScratchSet& sc, const GemmPlan& g, int M, int K) {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = M;
  a.K = K;
  a.n_tiles = g.n_tiles;
  a.m_tiles = g.m_tiles;
  a.k_frags = g.k_frags;
  a.ksplit = g.ksplit;
  a.partial = sc.gpart;
  a.counters = sc.gcnt;
  a.ssq_tiles = h->ssq_tiles;
  a.ldssq = h->Mmax;
  a.eps = h->cfg.rms_eps;
  return a;
}

#define AE_LAUNCH(call)                                      \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return hip_fail(h, e_, #call);     \
  } while (0)

// The time path: sinusoidal embeddings of t_k, the time MLP and every
// layer's modulation (scale/shift/gate) plus the final norm's, for all steps
// of a call.  It depends only on the step count and the weights, so its table
// is kept and recomputed only when the step count changes or weights load.
ae_status enqueue_tpath(ae_handle* h, int steps, hipStream_t s) {
  const int D = h->D, L = h->L;
  AE_LAUNCH(launch_tpath_sinusoid(h->e, steps, D, s));
  for (int r0 = 0; r0 < steps; r0 += 16) {
    const int mr = std::min(16, steps - r0);
    AE_LAUNCH(launch_gemv_rows(h->dt, h->e + static_cast<size_t>(r0) * D, D, mr, D, h->tw1, D, h->tb1,
                               D, h->z + static_cast<size_t>(r0) * D, D, 1, 1, 0, 0, 0, s));
    AE_LAUNCH(launch_gemv_rows(h->dt, h->z + static_cast<size_t>(r0) * D, D, mr, D, h->tw2, D, h->tb2,
                               D, h->c + static_cast<size_t>(r0) * D, D, 1, 1, 0, 0, 0, s));
    const int nm = h->nmod * D;
    AE_LAUNCH(launch_gemv_rows(h->dt, h->c + static_cast<size_t>(r0) * D, D, mr, D, h->mod_w, nm,
                               h->mod_b, nm, h->mod + static_cast<size_t>(r0) * L * nm,
                               L * nm, 0, L, static_cast<size_t>(D) * nm, nm, nm, s));
    AE_LAUNCH(launch_gemv_rows(h->dt, h->c + static_cast<size_t>(r0) * D, D, mr, D, h->fmod_w, 2 * D,
                               h->fmod_b, 2 * D, h->fmod + static_cast<size_t>(r0) * 2 * D, 2 * D, 0,
                               1, 0, 0, 0, s));
  }
  if (h->dit) {  // shift W of the attn1 (chunk 1), attn2 (chunk 4) and MLP (chunk 7) norms
    AE_LAUNCH(launch_shift_bias(h->dt, h->wqkv, h->sqkv, D, h->qkv_n, h->mod, steps, L, D, 9, 1, h->bq, s));
    AE_LAUNCH(launch_shift_bias(h->dt, h->wq2, h->sq2, D, h->qdim, h->mod, steps, L, D, 9, 4, h->bq2, s));
    AE_LAUNCH(launch_shift_bias(h->dt, h->wgu, h->sgu, D, 2 * h->F, h->mod, steps, L, D, 9, 7, h->bg, s));
  } else if (h->bq) {  // shift W of the attention (chunk 1) and MLP (chunk 4) norms
    AE_LAUNCH(launch_shift_bias(h->dt, h->wqkv, h->sqkv, D, h->qkv_n, h->mod, steps, L, D, 6, 1, h->bq, s));
    AE_LAUNCH(launch_shift_bias(h->dt, h->wgu, h->sgu, D, 2 * h->F, h->mod, steps, L, D, 6, 4, h->bg, s));
  }
  return AE_OK;
}

// Enqueue the N Euler steps of one denoise call, reading and writing the
// static buffers; used both directly and under stream capture.
ae_status enqueue_loop_tiled(ae_handle* h, const ScratchSet& sc, int batch, int steps, hipStream_t s);

ae_status enqueue_loop(ae_handle* h, const ScratchSet& sc, int batch, int steps, hipStream_t s) {
  if (h->tiled) return enqueue_loop_tiled(h, sc, batch, steps, s);
  const int D = h->D, L = h->L, M = batch * h->T;
  const size_t kv_layer = static_cast<size_t>(h->Bmax) * h->Hkv * h->S_max * h->dh * h->esz;
  const LayerPlans lp = plan_layer(h, M);
  const AttnPlan ap = plan_attention_batched(h, batch, h->span);
  const float dt = -1.0f / static_cast<float>(steps);
  for (int k = 0; k < steps; ++k) {
    AE_LAUNCH(launch_action_in(h->x, M, h->A, h->w_in, h->b_in, h->h, D, h->ssq, h->Mmax, s));
    for (int l = 0; l < L; ++l) {
      const float* md = h->mod + (static_cast<size_t>(k) * L + l) * 6 * D;
      char* kc = static_cast<char*>(h->kcache) + l * kv_layer;
      char* vc = static_cast<char*>(h->vtcache) + l * kv_layer;

      GemmArgs g = base_gemm(h, sc, lp.qkv, M, D);
      g.A = h->h; g.lda = D; g.W = h->wqkv + l * h->sqkv;
      g.ssq = h->ssq; g.scale = md; g.shift = md + D;
      g.q = h->q; g.ldq = h->qdim; g.kcache = kc; g.vtcache = vc; g.n_valid = h->n_valid;
      g.rope_cos = h->rope_cos; g.rope_sin = h->rope_sin;
      g.T = h->T; g.Hq = h->Hq; g.Hkv = h->Hkv; g.dh = h->dh; g.S_max = h->S_max;
      AE_LAUNCH(launch_gemm(h->dt, PRO_ADARMS, EPI_QKV, g, lp.qkv.blocks, s));

      AttnArgs at;
      std::memset(&at, 0, sizeof(at));
      at.q = h->q; at.ldq = h->qdim; at.kcache = kc; at.vtcache = vc; at.S_max = h->S_max;
      at.n_valid = h->n_valid; at.o = h->o; at.ldo = h->qdim;
      at.T = h->T; at.Hq = h->Hq; at.Hkv = h->Hkv; at.dh = h->dh; at.n_act = h->T;
      at.batch = batch; at.n_qg = ap.n_qg; at.nsplit = ap.nsplit; at.kc_len = ap.kc_len;
      at.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->dh)));
      at.partial = sc.apart; at.counters = sc.acnt;
      AE_LAUNCH(launch_attention(h->dt, at, s));

      g = base_gemm(h, sc, lp.o, M, h->qdim);
      g.A = h->o; g.lda = h->qdim; g.W = h->wo + l * h->so;
      g.h = h->h; g.ldh = D; g.gate = md + 2 * D; g.ssq_out = h->ssq;
      AE_LAUNCH(launch_gemm(h->dt, PRO_NONE, EPI_RESID, g, lp.o.blocks, s));

      g = base_gemm(h, sc, lp.gu, M, D);
      g.A = h->h; g.lda = D; g.W = h->wgu + l * h->sgu;
      g.ssq = h->ssq; g.scale = md + 3 * D; g.shift = md + 4 * D;
      g.out = h->act; g.ldo = h->F;
      AE_LAUNCH(launch_gemm(h->dt, PRO_ADARMS, EPI_GELU, g, lp.gu.blocks, s));

      g = base_gemm(h, sc, lp.d, M, h->F);
      g.A = h->act; g.lda = h->F; g.W = h->wd + l * h->sd;
      g.h = h->h; g.ldh = D; g.gate = md + 5 * D; g.ssq_out = h->ssq;
      AE_LAUNCH(launch_gemm(h->dt, PRO_NONE, EPI_RESID, g, lp.d.blocks, s));
    }
    const float* fm = h->fmod + static_cast<size_t>(k) * 2 * D;
    AE_LAUNCH(launch_action_out(h->x, M, h->A, h->h, D, fm, fm + D, h->cfg.rms_eps, h->w_out,
                                h->b_out, dt, s));
  }
  return AE_OK;
}

// The N Euler steps on the batched tiled path.  Per layer: (fp8: adaRMS rows
// and their per-request codes), QKV + RoPE, attention, O-proj + gated
// residual, (fp8: adaRMS rows and codes), gate/up + gelu, (fp8: codes of the
// activations), down + gated residual.  In bf16 the norms run after the
// product: the residual epilogues (and action-in) write the shadow
// ha = bf16(h (1 + scale)) of the next norm with h's row sums of squares, and
// QKV / gate-up finish with 1 / rms and the precomputed shift W.
ae_status enqueue_loop_dit(ae_handle* h, const ScratchSet& sc, int batch, int steps, hipStream_t s);

ae_status enqueue_loop_tiled(ae_handle* h, const ScratchSet& sc, int batch, int steps, hipStream_t s) {
  if (h->dit) return enqueue_loop_dit(h, sc, batch, steps, s);
  const int D = h->D, L = h->L, F = h->F, M = batch * h->T;
  const size_t kv_layer = static_cast<size_t>(h->Bmax) * h->Hkv * h->S_max * h->dh * h->esz;
  const TPlans tp = plan_tlayer(h, M);
  const AttnPlan ap = plan_attention_batched(h, batch, h->span);
  const float dt = -1.0f / static_cast<float>(steps);
  const float eps = h->cfg.rms_eps;
  const bool f8 = h->fp8;
  const size_t ob = f8 ? 1 : 2;  // operand bytes
  uint8_t* ub8 = static_cast<uint8_t*>(h->ubuf);
  // fp8: the adaRMS input of a QKV / gate-up product as e4m3 codes
  auto norm_rows = [&](const float* sc, const float* sh) -> ae_status {
    if (h->rowwise) {  // each row its own scale: norm and codes in one pass
      AE_LAUNCH(launch_rownorm_quant(h->h, M, D, sc, sh, eps, h->rrow, ub8, h->sxrow, s));
      return AE_OK;
    }
    AE_LAUNCH(launch_rownorm(h->h, M, D, sc, sh, eps, h->rrow, h->rowmax, s));
    AE_LAUNCH(launch_quant(nullptr, h->h, h->rrow, sc, sh, M, D, h->T, h->rowmax, 1, h->Mmax, ub8,
                           h->sxrow, s));
    return AE_OK;
  };
  // prefetch workgroups of a GEMM launch (on the CUs its tiles leave free):
  // layer ll's part of a K or V cache for these requests
  auto prefetch_cache = [&](TGemmArgs& g, const void* cache, int ll, int blocks) {
    g.pf_blocks = std::max(0, kTargetBlocks - blocks);
    g.pf[0] = reinterpret_cast<const uint4*>(static_cast<const char*>(cache) + static_cast<size_t>(ll) * kv_layer);
    g.pf_n4[0] = static_cast<int>(static_cast<size_t>(batch) * h->Hkv * h->S_max * h->dh * h->esz / 16);
  };
  uint16_t* ha = static_cast<uint16_t*>(h->ha);
  // the bf16 norm-after-product inputs of a QKV / gate-up product
  auto post_norm = [&](TGemmArgs& g, const float* bias) {
    g.A = ha; g.lda_bytes = static_cast<size_t>(D) * 2;
    g.bias = bias; g.ssq = h->ssq; g.ldssq = h->Mmax; g.ssq_tiles = h->ssq_tiles; g.eps = eps;
  };
  // ... and the outputs of a residual epilogue feeding one
  auto resid_out = [&](TGemmArgs& g, const float* next_scale) {
    g.ssq = h->ssq; g.ldssq = h->Mmax; g.nsc = next_scale; g.ha = ha;
  };
  for (int k = 0; k < steps; ++k) {
    const float* md0 = h->mod + static_cast<size_t>(k) * L * 6 * D;
    AE_LAUNCH(launch_action_in(h->x, M, h->A, h->w_in, h->b_in, h->h, D, h->ssq, h->Mmax, s,
                               f8 ? nullptr : ha, f8 ? nullptr : md0));
    for (int l = 0; l < L; ++l) {
      const float* md = h->mod + (static_cast<size_t>(k) * L + l) * 6 * D;
      const size_t it = static_cast<size_t>(k) * L + l;
      char* kc = static_cast<char*>(h->kcache) + l * kv_layer;
      char* vc = static_cast<char*>(h->vtcache) + l * kv_layer;
      if (f8) {
        ae_status r = norm_rows(md, md + D);
        if (r != AE_OK) return r;
      }

      // row-wise fp8: this layer's weight scales per packed column
      const float* swl = h->rowwise ? h->swc + l * h->swc_layer : nullptr;
      TGemmArgs g = base_tgemm(h, sc, tp.qkv, M, h->qkv_n, D);
      g.A = h->ubuf; g.lda_bytes = D * ob; g.W = h->wqkv + l * h->sqkv; g.sw = h->wsc + 6 * l;
      g.swc = swl;
      if (!f8) post_norm(g, h->bq + it * h->qkv_n);  // (bf16: A = the norm shadow)
      g.q = h->q; g.ldq = h->qdim; g.kcache = kc; g.vtcache = vc; g.n_valid = h->n_valid;
      g.rope_cos = h->rope_cos; g.rope_sin = h->rope_sin;
      g.T = h->T; g.Hq = h->Hq; g.Hkv = h->Hkv; g.dh = h->dh; g.S_max = h->S_max;
      AE_LAUNCH(launch_tgemm(tp.op, EPI_QKV, g, tp.qkv.blocks, s));

      AttnArgs at;
      std::memset(&at, 0, sizeof(at));
      at.q = h->q; at.ldq = h->qdim; at.kcache = kc; at.vtcache = vc; at.S_max = h->S_max;
      at.n_valid = h->n_valid; at.o = h->o; at.ldo = h->qdim;
      at.T = h->T; at.Hq = h->Hq; at.Hkv = h->Hkv; at.dh = h->dh; at.n_act = h->T;
      at.batch = batch; at.n_qg = ap.n_qg; at.nsplit = ap.nsplit; at.kc_len = ap.kc_len;
      at.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->dh)));
      at.partial = sc.apart; at.counters = sc.acnt;
      // warm the last-level cache with this layer's O / gate-up / down
      // weights and the next layer's QKV weights while attention runs
      at.pf_blocks = kPrefetchBlocks;
      at.pf[0] = h->wo + l * h->so;
      at.pf_n4[0] = static_cast<int>(static_cast<size_t>(h->qdim) * D * (h->fp8o ? 1 : 2) / 16);
      at.pf[1] = h->wgu + l * h->sgu;
      at.pf_n4[1] = static_cast<int>(static_cast<size_t>(D) * 2 * F * ob / 16);
      at.pf[2] = h->wd + l * h->sd;
      at.pf_n4[2] = static_cast<int>(static_cast<size_t>(F) * D * ob / 16);
      at.pf[3] = h->wqkv + ((l + 1) % L) * h->sqkv;
      at.pf_n4[3] = static_cast<int>(static_cast<size_t>(D) * h->qkv_n * ob / 16);
      AE_LAUNCH(launch_attention(h->dt, at, s));

      g = base_tgemm(h, sc, tp.o, M, D, h->qdim);
      g.A = h->o; g.lda_bytes = static_cast<size_t>(h->qdim) * 2; g.W = h->wo + l * h->so;
      if (h->fp8o) {  // the attention output's codes, a scale per row
        AE_LAUNCH(launch_quant_bf16_rows(static_cast<const uint16_t*>(h->o), M, h->qdim, ub8, h->sxrow, s));
        g.A = h->ubuf; g.lda_bytes = static_cast<size_t>(h->qdim);
        g.swc = swl + h->qkv_n + 2 * F + D;
      }
      // the next layer's K cache of these requests into the last-level
      // cache on the CUs the O-proj tiles leave free (its V: beside down)
      prefetch_cache(g, h->kcache, (l + 1) % L, tp.o.blocks);
      g.h = h->h; g.ldh = D; g.gate = md + 2 * D;
      if (!f8) resid_out(g, md + 3 * D);
      AE_LAUNCH(launch_tgemm(h->fp8o ? OP_FP8 : OP_BF16, EPI_RESID, g, tp.o.blocks, s));

      if (f8) {
        ae_status r = norm_rows(md + 3 * D, md + 4 * D);
        if (r != AE_OK) return r;
      }
      g = base_tgemm(h, sc, tp.gu, M, 2 * F, D);
      g.A = h->ubuf; g.lda_bytes = D * ob; g.W = h->wgu + l * h->sgu; g.sw = h->wsc + 6 * l + 3;
      g.swc = swl ? swl + h->qkv_n : nullptr;
      g.out = h->act; g.ldo = F; g.rowmax = h->rowmax; g.ldp = h->Mmax;
      if (!f8) post_norm(g, h->bg + it * 2 * F);
      AE_LAUNCH(launch_tgemm(tp.op, EPI_GELU, g, tp.gu.blocks, s));
      if (f8)
        AE_LAUNCH(launch_quant(static_cast<const float*>(h->act), nullptr, nullptr, nullptr, nullptr, M, F,
                               h->rowwise ? 1 : h->T, h->rowmax, tp.gu.n_tiles, h->Mmax, ub8, h->sxrow, s));

      g = base_tgemm(h, sc, tp.d, M, D, F);
      g.A = f8 ? h->ubuf : h->act; g.lda_bytes = F * ob; g.W = h->wd + l * h->sd;
      prefetch_cache(g, h->vtcache, (l + 1) % L, tp.d.blocks);
      g.sw = h->wsc + 6 * l + 5;
      g.swc = swl ? swl + h->qkv_n + 2 * F : nullptr;
      g.h = h->h; g.ldh = D; g.gate = md + 5 * D;
      // the next layer's attention norm (the last layer's h goes to the
      // final norm, which reads h itself)
      if (!f8) resid_out(g, l + 1 < L ? md + 6 * D : nullptr);
      AE_LAUNCH(launch_tgemm(tp.op, EPI_RESID, g, tp.d.blocks, s));
    }
    const float* fm = h->fmod + static_cast<size_t>(k) * 2 * D;
    AE_LAUNCH(launch_action_out(h->x, M, h->A, h->h, D, fm, fm + D, h->cfg.rms_eps, h->w_out,
                                h->b_out, dt, s));
  }
  return AE_OK;
}

// The N Euler steps with the DiT-style block (MolmoBot PR Part 2: the block
// hands the cached context K/V to its second attention; its correctness
// table lists cross_attn and self_attn apart), on the batched tiled path in
// bf16.  Per layer, with the nine modulation chunks (scale, shift, gate of
// attn1, attn2 and the MLP):
//   QKV + RoPE of adaRMS_1(h) into the action-only cache; attn1 over it;
//   O-proj + gate_1 residual;
//   q2 + RoPE of adaRMS_2(h); attn2 over the visible prefix alone;
//   o2 + gate_2 residual;
//   gate/up of adaRMS_3(h) + gelu; down + gate_3 residual.
// Action token t of request b sits at position n_b + t in both attentions
// (only differences matter in attn1).  The norms run after the products as
// in the joint block: each residual epilogue writes the next norm's
// modulated shadow and row sums of squares.
ae_status enqueue_loop_dit(ae_handle* h, const ScratchSet& sc, int batch, int steps, hipStream_t s) {
  const int D = h->D, L = h->L, F = h->F, M = batch * h->T, NM = 9 * D;
  const size_t kv_layer = static_cast<size_t>(h->Bmax) * h->Hkv * h->S_max * h->dh * h->esz;
  const size_t self_layer = static_cast<size_t>(h->Bmax) * h->Hkv * h->S_self * h->dh * h->esz;
  const TPlans tp = plan_tlayer(h, M);
  const AttnPlan a_self = plan_attention_batched(h, batch, 0);
  const AttnPlan a_cross = plan_attention_batched(h, batch, h->span);
  const float dt = -1.0f / static_cast<float>(steps);
  const float eps = h->cfg.rms_eps;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->dh)));
  uint16_t* ha = static_cast<uint16_t*>(h->ha);
  auto post_norm = [&](TGemmArgs& g, const float* bias) {
    g.A = ha; g.lda_bytes = static_cast<size_t>(D) * 2;
    g.bias = bias; g.ssq = h->ssq; g.ldssq = h->Mmax; g.ssq_tiles = h->ssq_tiles; g.eps = eps;
  };
  auto resid_out = [&](TGemmArgs& g, const float* next_scale) {
    g.ssq = h->ssq; g.ldssq = h->Mmax; g.nsc = next_scale; g.ha = ha;
  };
  // queries (q or q2, RoPE at n_b + t) and, with a cache, the action rows' K/V
  auto qkv_args = [&](TGemmArgs& g, void* kc, void* vc, const int* nv, int S, int Hkv) {
    g.q = h->q; g.ldq = h->qdim; g.kcache = kc; g.vtcache = vc; g.n_valid = nv;
    g.rope_cos = h->rope_cos; g.rope_sin = h->rope_sin;
    g.T = h->T; g.Hq = h->Hq; g.Hkv = Hkv; g.dh = h->dh; g.S_max = S;
  };
  struct Pf {
    const uint4* p;
    int n4;
  };
  auto attention = [&](const AttnPlan& ap, const void* kc, const void* vc, int S, const int* nv, int n_act,
                       std::initializer_list<Pf> pf) -> ae_status {
    AttnArgs at;
    std::memset(&at, 0, sizeof(at));
    at.q = h->q; at.ldq = h->qdim; at.kcache = kc; at.vtcache = vc; at.S_max = S;
    at.n_valid = nv; at.n_act = n_act; at.o = h->o; at.ldo = h->qdim;
    at.T = h->T; at.Hq = h->Hq; at.Hkv = h->Hkv; at.dh = h->dh;
    at.batch = batch; at.n_qg = ap.n_qg; at.nsplit = ap.nsplit; at.kc_len = ap.kc_len;
    at.scale_log2 = scale_log2;
    at.partial = sc.apart; at.counters = sc.acnt;
    // warm the last-level cache with the next products' weights
    at.pf_blocks = kPrefetchBlocks;
    int i = 0;
    for (const Pf& w : pf) {
      at.pf[i] = w.p;
      at.pf_n4[i++] = w.n4;
    }
    AE_LAUNCH(launch_attention(h->dt, at, s));
    return AE_OK;
  };
  const int o_n4 = static_cast<int>(static_cast<size_t>(h->qdim) * D * 2 / 16);
  const int q2_n4 = o_n4;
  const int gu_n4 = static_cast<int>(static_cast<size_t>(D) * 2 * F * 2 / 16);
  const int d_n4 = static_cast<int>(static_cast<size_t>(F) * D * 2 / 16);
  const int qkv_n4 = static_cast<int>(static_cast<size_t>(D) * h->qkv_n * 2 / 16);
  for (int k = 0; k < steps; ++k) {
    const float* md0 = h->mod + static_cast<size_t>(k) * L * NM;
    AE_LAUNCH(launch_action_in(h->x, M, h->A, h->w_in, h->b_in, h->h, D, h->ssq, h->Mmax, s, ha, md0));
    for (int l = 0; l < L; ++l) {
      const float* md = md0 + static_cast<size_t>(l) * NM;
      const size_t it = static_cast<size_t>(k) * L + l;
      char* ks = static_cast<char*>(h->kself) + l * self_layer;
      char* vs = static_cast<char*>(h->vtself) + l * self_layer;
      const char* kc = static_cast<const char*>(h->kcache) + l * kv_layer;
      const char* vc = static_cast<const char*>(h->vtcache) + l * kv_layer;

      // attn1: the action tokens among themselves
      TGemmArgs g = base_tgemm(h, sc, tp.qkv, M, h->qkv_n, D);
      g.W = h->wqkv + l * h->sqkv;
      post_norm(g, h->bq + it * h->qkv_n);
      qkv_args(g, ks, vs, h->zeros, h->S_self, h->Hkv);
      AE_LAUNCH(launch_tgemm(OP_BF16, EPI_QKV, g, tp.qkv.blocks, s));
      ae_status r = attention(a_self, ks, vs, h->S_self, h->zeros, h->T,
                              {{h->wo + l * h->so, o_n4}, {h->wq2 + l * h->sq2, q2_n4}});
      if (r != AE_OK) return r;
      g = base_tgemm(h, sc, tp.o, M, D, h->qdim);
      g.A = h->o; g.lda_bytes = static_cast<size_t>(h->qdim) * 2; g.W = h->wo + l * h->so;
      g.h = h->h; g.ldh = D; g.gate = md + 2 * D;
      resid_out(g, md + 3 * D);
      AE_LAUNCH(launch_tgemm(OP_BF16, EPI_RESID, g, tp.o.blocks, s));

      // attn2: the action queries over the visible prefix
      g = base_tgemm(h, sc, tp.q2, M, h->qdim, D);
      g.W = h->wq2 + l * h->sq2;
      post_norm(g, h->bq2 + it * h->qdim);
      qkv_args(g, nullptr, nullptr, h->n_valid, h->S_max, 0);
      AE_LAUNCH(launch_tgemm(OP_BF16, EPI_QKV, g, tp.q2.blocks, s));
      r = attention(a_cross, kc, vc, h->S_max, h->n_valid, 0,
                    {{h->wo2 + l * h->so, o_n4}, {h->wgu + l * h->sgu, gu_n4}, {h->wd + l * h->sd, d_n4},
                     {h->wqkv + ((l + 1) % L) * h->sqkv, qkv_n4}});
      if (r != AE_OK) return r;
      g = base_tgemm(h, sc, tp.o, M, D, h->qdim);
      g.A = h->o; g.lda_bytes = static_cast<size_t>(h->qdim) * 2; g.W = h->wo2 + l * h->so;
      g.h = h->h; g.ldh = D; g.gate = md + 5 * D;
      resid_out(g, md + 6 * D);
      AE_LAUNCH(launch_tgemm(OP_BF16, EPI_RESID, g, tp.o.blocks, s));

      // MLP
      g = base_tgemm(h, sc, tp.gu, M, 2 * F, D);
      g.W = h->wgu + l * h->sgu;
      g.out = h->act; g.ldo = F;
      post_norm(g, h->bg + it * 2 * F);
      AE_LAUNCH(launch_tgemm(OP_BF16, EPI_GELU, g, tp.gu.blocks, s));
      g = base_tgemm(h, sc, tp.d, M, D, F);
      g.A = h->act; g.lda_bytes = static_cast<size_t>(F) * 2; g.W = h->wd + l * h->sd;
      g.h = h->h; g.ldh = D; g.gate = md + 8 * D;
      resid_out(g, l + 1 < L ? md + NM : nullptr);  // the next layer's attn1 norm
      AE_LAUNCH(launch_tgemm(OP_BF16, EPI_RESID, g, tp.d.blocks, s));
    }
    const float* fm = h->fmod + static_cast<size_t>(k) * 2 * D;
    AE_LAUNCH(launch_action_out(h->x, M, h->A, h->h, D, fm, fm + D, h->cfg.rms_eps, h->w_out,
                                h->b_out, dt, s));
  }
  return AE_OK;
}

PersistArgs persist_args(const ae_handle* h, const ScratchSet& sc, int batch, int steps) {
  PersistArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = batch * h->T; a.D = h->D; a.L = h->L; a.n_steps = steps; a.T = h->T; a.A = h->A;
  a.Hq = h->Hq; a.Hkv = h->Hkv; a.dh = h->dh; a.F = h->F; a.S_max = h->S_max; a.qdim = h->qdim;
  a.ssq_tiles = h->ssq_tiles; a.ldssq = h->Mmax; a.batch = batch; a.G = h->G;
  a.eps = h->cfg.rms_eps;
  a.dt = -1.0f / static_cast<float>(steps);
  a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->dh)));
  a.wqkv = h->wqkv; a.wo = h->wo; a.wgu = h->wgu; a.wd = h->wd;
  a.sqkv = h->sqkv; a.so = h->so; a.sgu = h->sgu; a.sd = h->sd;
  a.win_p = h->win_p; a.wout_p = h->wout_p; a.a_frags = h->a_frags; a.a_blocks = h->a_blocks;
  a.b_in = h->b_in; a.b_out = h->b_out; a.mod = h->mod; a.fmod = h->fmod;
  a.kcache = h->kcache; a.vtcache = h->vtcache;
  a.kv_layer = static_cast<size_t>(h->Bmax) * h->Hkv * h->S_max * h->dh;
  a.n_valid = h->n_valid; a.rope_cos = h->rope_cos; a.rope_sin = h->rope_sin;
  a.x = h->x; a.h = h->h; a.ssq = h->ssq; a.q = h->q; a.o = h->o; a.act = h->act;
  a.ha = h->ha; a.bq = h->bq; a.bg = h->bg; a.qkv_n = h->qkv_n;
  a.gpart = sc.gpart; a.gcnt = sc.gcnt; a.apart = sc.apart;
  a.flags = sc.flags; a.err = h->derr; a.genp = sc.genp;
  a.pcnt = sc.pcnt;
  const PersistPlans pp = plan_persist(h);
  a.pq = pp.q; a.po = pp.o; a.pg = pp.g; a.pd = pp.d;
  const AttnPlan ap = plan_attention(h, batch, h->span, kTileM, kPersistMaxSplits);
  a.n_qg = ap.n_qg; a.nsplit = ap.nsplit; a.kc_len = ap.kc_len;
  a.n_acnt = ap.items;
  a.acnt = sc.pcnt + pp.q.n_tiles + pp.o.n_tiles + pp.g.n_tiles + pp.d.n_tiles;
  return a;
}

// The scratch a call at batch b and prefix span `span` needs on the
// whole-call path (persist) or the per-phase path; any_span bounds the
// attention's key splits over every span up to the capacity instead.
ScratchNeed scratch_need(const ae_handle* h, int b, int span, bool persist, bool any_span) {
  ScratchNeed n;
  if (persist) {
    const AttnPlan pa = plan_attention(h, b, span, kTileM, kPersistMaxSplits);
    const int nsp = any_span ? max_attention_splits(h, pa.items, kPersistMaxSplits) : pa.nsplit;
    if (nsp > 1) n.afl = attention_partial_floats(h->dh, pa.items, nsp, kTileM);
    const PersistPlans pp = plan_persist(h);
    n.pcnt = pa.items;
    for (const PGemm* g : {&pp.q, &pp.o, &pp.g, &pp.d}) {
      if (g->ksplit > 1)  // (value, generation) packets: two words per value
        n.gfl = std::max(n.gfl, 2 * static_cast<size_t>(g->n_tiles) * g->ksplit * kTileM * kTileN);
      n.pcnt += g->n_tiles;
    }
    n.flags = static_cast<size_t>(h->G);
    return n;
  }
  if (h->tiled) {
    const TPlans tp = plan_tlayer(h, b * h->T);
    for (const TGemmPlan* g : {&tp.qkv, &tp.o, &tp.gu, &tp.d, &tp.q2}) {
      if (g == &tp.q2 && !h->dit) continue;
      n.gfl = std::max(n.gfl, tgemm_partial_floats(*g));
      n.gcn = std::max(n.gcn, static_cast<size_t>(g->m_tiles) * g->n_tiles);
    }
  } else {
    const LayerPlans lp = plan_layer(h, b * h->T);
    for (const GemmPlan* g : {&lp.qkv, &lp.o, &lp.gu, &lp.d}) {
      n.gfl = std::max(n.gfl, gemm_scratch_floats(*g));
      n.gcn = std::max(n.gcn, static_cast<size_t>(g->m_tiles) * g->n_tiles);
    }
  }
  const AttnPlan ap = plan_attention_batched(h, b, span);
  const int ns = any_span ? max_attention_splits(h, ap.items, attention_max_splits(ap.items)) : ap.nsplit;
  if (ns > 1) n.afl = attention_partial_floats(h->dh, ap.items, ns, attention_rows_per_item());
  n.acn = static_cast<size_t>(ap.items);
  return n;
}

void destroy_entry(GraphEntry& g) {
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  if (g.done) (void)hipEventDestroy(g.done);
  g = GraphEntry{};
}

// Destroy the evicted graphs whose last replay has completed (a non-blocking
// event query each).
void reap_retired(ae_handle* h) {
  std::vector<GraphEntry> keep;
  for (auto& g : h->retired) {
    if (!g.done || hipEventQuery(g.done) == hipSuccess) destroy_entry(g);
    else keep.push_back(g);
  }
  (void)hipGetLastError();
  h->retired.swap(keep);
}

// Every graph, cached or retired (the caller has synchronised the device).
void drop_graphs(ae_handle* h) {
  for (auto& g : h->graphs.drain()) destroy_entry(g);
  for (auto& g : h->retired) destroy_entry(g);
  h->retired.clear();
}

struct WeightSpec {
  std::string name;
  std::vector<long long> shape;
};

std::vector<WeightSpec> weight_specs(const ae_handle* h) {
  const long long D = h->D, A = h->A, F = h->F, qd = h->qdim, kd = h->kvdim;
  std::vector<WeightSpec> v = {
      {"time_mlp.1.w", {D, D}}, {"time_mlp.1.b", {D}}, {"time_mlp.2.w", {D, D}},
      {"time_mlp.2.b", {D}},    {"action_in.w", {A, D}}, {"action_in.b", {D}},
      {"action_out.w", {D, A}}, {"action_out.b", {A}},   {"final_mod.w", {D, 2 * D}},
      {"final_mod.b", {2 * D}},
  };
  for (int l = 0; l < h->L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    v.push_back({p + "q", {D, qd}});
    v.push_back({p + "k", {D, kd}});
    v.push_back({p + "v", {D, kd}});
    v.push_back({p + "o", {qd, D}});
    v.push_back({p + "gate", {D, F}});
    v.push_back({p + "up", {D, F}});
    v.push_back({p + "down", {F, D}});
    v.push_back({p + "mod.w", {D, h->nmod * D}});
    v.push_back({p + "mod.b", {h->nmod * D}});
    if (h->dit) {
      v.push_back({p + "q2", {D, qd}});
      v.push_back({p + "o2", {qd, D}});
    }
    if (h->Dc > 0) {
      v.push_back({p + "ctx_k", {h->Dc, kd}});
      v.push_back({p + "ctx_v", {h->Dc, kd}});
    }
  }
  if (h->Sd > 0) {
    v.push_back({"state_in.w", {h->Sd, h->Dc}});
    v.push_back({"state_in.b", {h->Dc}});
  }
  return v;
}

std::string shape_str(const long long* s, int n) {
  std::string r = "[";
  for (int i = 0; i < n; ++i) r += (i ? "," : "") + std::to_string(s[i]);
  return r + "]";
}

// Parts of a scratch set laid out from `base` (nullptr: sizes only), each
// 256-byte aligned, the packet generation base first: its place must not move
// between calls that share the memory, since every launch continues from the
// range the previous one used.  Returns the bytes used.
size_t carve(char* base, const ScratchNeed& n, ScratchSet* sc) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (std::max<size_t>(bytes, 4) + 255) / 256 * 256;
    return p;
  };
  sc->genp = reinterpret_cast<uint32_t*>(take(8));
  sc->flags = reinterpret_cast<int*>(take(n.flags * 4));
  sc->pcnt = reinterpret_cast<int*>(take(n.pcnt * 4));
  sc->gcnt = reinterpret_cast<int*>(take(n.gcn * 4));
  sc->acnt = reinterpret_cast<int*>(take(n.acn * 4));
  sc->gpart = reinterpret_cast<float*>(take(n.gfl * 4));
  sc->apart = reinterpret_cast<float*>(take(n.afl * 4));
  return off;
}

// Checks shared by ae_denoise and ae_denoise_static (before any state change).
ae_status check_denoise(ae_handle* h, const float* noise, int batch, int steps, const float* actions_out) {
  if (!noise || !actions_out) return fail(h, AE_ERR_INVALID_ARGUMENT, "null noise or actions_out");
  if (!h->weights_loaded) return fail(h, AE_ERR_NOT_READY, "weights not loaded");
  if (h->prefix_batch < 0) return fail(h, AE_ERR_NOT_READY, "prefix K/V not set");
  if (batch != h->prefix_batch)
    return fail(h, AE_ERR_SHAPE_MISMATCH,
                "batch " + std::to_string(batch) + " differs from the prefix batch " +
                    std::to_string(h->prefix_batch));
  if (steps < 1 || steps > h->Nmax)
    return fail(h, AE_ERR_INVALID_ARGUMENT,
                "steps " + std::to_string(steps) + " outside [1, " + std::to_string(h->Nmax) + "]");
  return AE_OK;
}

// The time-path table for `steps`, rebuilt only when the step count changed.
ae_status ensure_tpath(ae_handle* h, int steps, hipStream_t st) {
  if (h->table_steps == steps) return AE_OK;
  h->table_steps = -1;
  ae_status s = enqueue_tpath(h, steps, st);
  if (s != AE_OK) return s;
  h->table_steps = steps;
  return AE_OK;
}

// ---------------------------------------------------------------------------
// The scratch of ae_denoise_static, for callers that cannot allocate: a
// static device array of kStaticScratchBytes in this library's code object.
// Every GPU the library runs on holds its own copy until the process ends;
// its address on a device is looked up once, in ae_create, with that device
// current.  Calls on one device share it (and its contents from the last
// call): those calls must not overlap.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = static_cast<size_t>(24) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// Look up this device's address of `scratch` (once per device; the device
// must be current).  A failure leaves it unset: ae_denoise_static then
// reports AE_ERR_HIP.
void register_static_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (g_static_ptr[dev]) return;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) g_static_ptr[dev] = p;
  else (void)hipGetLastError();
}

void* static_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_static_mu);
  return g_static_ptr[dev];
}

}  // namespace

extern "C" {

const char* ae_status_string(int s) {
  switch (s) {
    case AE_OK: return "ok";
    case AE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case AE_ERR_SHAPE_MISMATCH: return "shape mismatch";
    case AE_ERR_NOT_READY: return "not ready";
    case AE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case AE_ERR_UNSUPPORTED: return "unsupported";
    case AE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ae_last_error(const ae_handle* h) { return h ? h->err.c_str() : "null handle"; }

ae_status ae_get_stats(const ae_handle* h, ae_stats* out) {
  if (!h || !out) return AE_ERR_INVALID_ARGUMENT;
  *out = h->stats;
  // launches whose waits timed out: the running count the counter fill
  // keeps, plus the last launch's flag if it is raised
  int derr[2] = {0, 0};
  if (h->derr && hipMemcpy(derr, h->derr, sizeof(derr), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    derr[0] = -1;
  }
  out->device_errors = derr[0] < 0 ? -1 : derr[1] + (derr[0] != 0);
  out->persistent = h->G > 0 ? h->G : 0;
  out->graphs_cached = h->graphs.size();
  out->prefix_bucket = h->span;
  return AE_OK;
}

void ae_destroy(ae_handle* h) {
  if (!h) return;
  if (h->cap_stream) (void)hipStreamSynchronize(h->cap_stream);
  (void)hipDeviceSynchronize();
  drop_graphs(h);
  for (auto& b : h->bufs) (void)hipFree(b.p);
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  delete h;
}

ae_status ae_create(const ae_config* cfg, ae_handle** out) {
  if (!out) return AE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (!cfg) return AE_ERR_INVALID_ARGUMENT;
  {
    std::string m = validate_config(cfg);
    if (!m.empty()) {
      std::fprintf(stderr, "ae_create: %s\n", m.c_str());
      return AE_ERR_INVALID_ARGUMENT;
    }
    m = unsupported_config(cfg);
    if (!m.empty()) {
      std::fprintf(stderr, "ae_create: %s\n", m.c_str());
      return AE_ERR_UNSUPPORTED;
    }
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return AE_ERR_HIP;
  }

  ae_handle* h = new ae_handle();
  h->cfg = *cfg;
  h->dt = cfg->act_dtype == AE_BF16 ? DT_BF16 : DT_F32;
  h->esz = h->dt == DT_BF16 ? 2 : 4;
  h->L = cfg->n_layers; h->D = cfg->width; h->Hq = cfg->n_q_heads; h->Hkv = cfg->n_kv_heads;
  h->dh = cfg->head_dim; h->F = cfg->mlp_dim; h->T = cfg->action_horizon; h->A = cfg->action_dim;
  h->Pmax = cfg->max_prefix_len; h->Bmax = cfg->max_batch; h->Nmax = cfg->max_steps;
  h->span = h->Pmax;
  h->graphs = LruCache<CallKey, GraphEntry>(cfg->use_graphs ? cfg->graph_cache_size : 0);
  h->S_max = (h->Pmax + h->T + 63) / 64 * 64;
  h->qdim = h->Hq * h->dh;
  h->kvdim = h->Hkv * h->dh;
  h->qkv_n = h->qdim + 2 * h->kvdim;
  h->ssq_tiles = h->D / 64;
  h->Mmax = h->Bmax * h->T;
  h->fp8 = cfg->proj_weight_dtype == AE_FP8_E4M3;
  h->rowwise = h->fp8 && cfg->fp8_rowwise;
  h->fp8o = h->fp8 && cfg->fp8_oproj;
  h->Dc = cfg->context_width;
  h->Sd = cfg->state_dim;
  h->dit = cfg->block_type == AE_BLOCK_DIT;
  h->nmod = h->dit ? 9 : 6;
  h->S_self = (h->T + 63) / 64 * 64;
  h->tiled = h->dt == DT_BF16 && h->D % 128 == 0 && h->qkv_n % 128 == 0 && (2 * h->F) % 128 == 0 &&
             h->qdim % 64 == 0 && h->F % 64 == 0;

  const int ks = kstep_of(h->dt);
  {
    // the persistent kernel needs every workgroup resident at once
    int dev = 0, coop = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
      h->device = dev;
      register_static_scratch(dev);
    }
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        coop && persist_blocks_per_cu(h->dt, h->dh) >= 1)
      h->G = std::min(cus, persist_max_grid());
    (void)hipGetLastError();
  }
  h->a_frags = (h->A + ks - 1) / ks;
  h->a_blocks = (h->A + 15) / 16;
  const size_t es = h->esz;
  const size_t D = h->D, L = h->L, F = h->F, A = h->A;
  ae_status st = AE_OK;
#define AE_ALLOC(ptr, bytes)                       \
  do {                                             \
    st = alloc(h, &(ptr), (bytes));                \
    if (st != AE_OK) { ae_destroy(h); return st; } \
  } while (0)

  AE_ALLOC(h->tw1, D * D * es);
  AE_ALLOC(h->tb1, D * es);
  AE_ALLOC(h->tw2, D * D * es);
  AE_ALLOC(h->tb2, D * es);
  AE_ALLOC(h->fmod_w, D * 2 * D * es);
  AE_ALLOC(h->fmod_b, 2 * D * es);
  const size_t NM = static_cast<size_t>(h->nmod) * D;  // modulation columns per layer
  AE_ALLOC(h->mod_w, L * D * NM * es);
  AE_ALLOC(h->mod_b, L * NM * es);
  AE_ALLOC(h->w_in, A * D * 4);
  AE_ALLOC(h->b_in, D * 4);
  AE_ALLOC(h->w_out, D * A * 4);
  AE_ALLOC(h->b_out, A * 4);
  h->sqkv = elems_packed(h->D, h->qkv_n, ks);
  h->so = elems_packed(h->qdim, h->D, ks);
  h->sgu = elems_packed(h->D, 2 * h->F, ks);
  h->sd = elems_packed(h->F, h->D, ks);
  AE_ALLOC(h->wqkv, L * h->sqkv * 16);
  AE_ALLOC(h->wo, L * h->so * 16);
  AE_ALLOC(h->wgu, L * h->sgu * 16);
  AE_ALLOC(h->wd, L * h->sd * 16);
  if (h->dit) {
    h->sq2 = elems_packed(h->D, h->qdim, ks);
    AE_ALLOC(h->wq2, L * h->sq2 * 16);
    AE_ALLOC(h->wo2, L * h->so * 16);
    const size_t sb = L * h->Bmax * h->Hkv * static_cast<size_t>(h->S_self) * h->dh * es;
    AE_ALLOC(h->kself, sb);
    AE_ALLOC(h->vtself, sb);
    AE_ALLOC(h->zeros, static_cast<size_t>(h->Bmax) * 4);
    AE_ALLOC(h->bq2, static_cast<size_t>(h->Nmax) * L * h->qdim * 4);
  }

  const size_t kvbytes = L * h->Bmax * h->Hkv * static_cast<size_t>(h->S_max) * h->dh * es;
  AE_ALLOC(h->kcache, kvbytes);
  AE_ALLOC(h->vtcache, kvbytes);
  AE_ALLOC(h->comp_idx, static_cast<size_t>(h->Bmax) * (h->Pmax > 0 ? h->Pmax : 1) * 4);
  AE_ALLOC(h->src_of, static_cast<size_t>(h->Bmax) * (h->Pmax > 0 ? h->Pmax : 1) * 4);
  AE_ALLOC(h->n_valid, static_cast<size_t>(h->Bmax) * 4);
  AE_ALLOC(h->rope_cos, static_cast<size_t>(h->Bmax) * h->T * (h->dh / 2) * 4);
  AE_ALLOC(h->rope_sin, static_cast<size_t>(h->Bmax) * h->T * (h->dh / 2) * 4);

  const size_t Mm = h->Mmax;
  AE_ALLOC(h->x, Mm * A * 4);
  AE_ALLOC(h->h, Mm * D * 4);
  AE_ALLOC(h->ssq, static_cast<size_t>(h->ssq_tiles) * Mm * 4);
  AE_ALLOC(h->q, Mm * h->qdim * es);
  AE_ALLOC(h->o, Mm * h->qdim * es);
  AE_ALLOC(h->act, Mm * F * (h->fp8 ? 4 : es));
  if (!h->fp8) {
    AE_ALLOC(h->ha, Mm * D * es);
    AE_ALLOC(h->bq, static_cast<size_t>(h->Nmax) * L * h->qkv_n * 4);
    AE_ALLOC(h->bg, static_cast<size_t>(h->Nmax) * L * 2 * F * 4);
  }
  if (h->tiled) {
    if (h->fp8) AE_ALLOC(h->ubuf, Mm * std::max({D, F, static_cast<size_t>(h->qdim)}));
    if (h->rowwise) {
      h->swc_layer = static_cast<size_t>(h->qkv_n) + 2 * F + 2 * D;
      AE_ALLOC(h->swc, L * h->swc_layer * 4);
      const size_t cols = static_cast<size_t>(h->qdim) + 2 * h->kvdim + 2 * F + 2 * D;
      AE_ALLOC(h->cmul, cols * 4);
      AE_ALLOC(h->csc, cols * 4);
    }
    AE_ALLOC(h->rrow, Mm * 4);
    AE_ALLOC(h->sxrow, Mm * 4);
    AE_ALLOC(h->rowmax, Mm * std::max<size_t>(1, 2 * F / 128) * 4);
    AE_ALLOC(h->wamax, L * 6 * 4);
    AE_ALLOC(h->wmul, L * 6 * 4);
    AE_ALLOC(h->wsc, L * 6 * 4);
  }
  AE_ALLOC(h->e, static_cast<size_t>(h->Nmax) * D * 4);
  AE_ALLOC(h->z, static_cast<size_t>(h->Nmax) * D * 4);
  AE_ALLOC(h->c, static_cast<size_t>(h->Nmax) * D * 4);
  AE_ALLOC(h->mod, static_cast<size_t>(h->Nmax) * L * NM * 4);
  AE_ALLOC(h->fmod, static_cast<size_t>(h->Nmax) * 2 * D * 4);

  // the largest call's scratch, over every batch, path and prefix bucket
  ScratchNeed need;
  if (h->Dc > 0) {  // the context products' K splits and tile counters, at any row count
    for (int m = 1; m <= h->Bmax * std::max(1, h->Pmax); ++m) {  // (every layer in one product)
      const TGemmPlan g = plan_tgemm(m, h->L * 2 * h->kvdim, h->Dc, tgemm_kc(OP_BF16), kTargetBlocks);
      need.gfl = std::max(need.gfl, tgemm_partial_floats(g));
      need.gcn = std::max(need.gcn, static_cast<size_t>(g.m_tiles) * g.n_tiles);
    }
  }
  for (int b = 1; b <= h->Bmax; ++b) {
    need.max_with(scratch_need(h, b, h->Pmax, false, true));
    if (h->G > 0 && b * h->T <= kTileM) need.max_with(scratch_need(h, b, h->Pmax, true, true));
  }
  AE_ALLOC(h->win_p, elems_packed(h->a_frags * ks, h->D, ks) * 16);
  AE_ALLOC(h->wout_p, elems_packed(h->D, 16 * h->a_blocks, ks) * 16);
  AE_ALLOC(h->own.flags, need.flags * 4);
  AE_ALLOC(h->own.pcnt, need.pcnt * 4);
  AE_ALLOC(h->derr, 8);
  AE_ALLOC(h->own.genp, 8);
  AE_ALLOC(h->own.gpart, need.gfl * 4);
  AE_ALLOC(h->own.gcnt, need.gcn * 4);
  AE_ALLOC(h->own.apart, need.afl * 4);
  AE_ALLOC(h->own.acnt, need.acn * 4);
  if (h->Dc > 0) {
    h->sctx = elems_packed(h->Dc, 2 * h->kvdim, ks);
    AE_ALLOC(h->wctx, L * h->sctx * 16);
    AE_ALLOC(h->pos_cos, static_cast<size_t>(h->Pmax + 1) * (h->dh / 2) * 4);
    AE_ALLOC(h->pos_sin, static_cast<size_t>(h->Pmax + 1) * (h->dh / 2) * 4);
    if (h->Sd > 0) {
      AE_ALLOC(h->st_w, static_cast<size_t>(h->Sd) * h->Dc * 2);
      AE_ALLOC(h->st_b, static_cast<size_t>(h->Dc) * 2);
      AE_ALLOC(h->st_h, static_cast<size_t>(h->Bmax) * h->Dc * 2);
      AE_ALLOC(h->st_key, static_cast<size_t>(h->Bmax) * 4);
    }
  }
#undef AE_ALLOC

  // zero everything once: counters must start at 0; caches and activations
  // hold finite values even where a kernel reads a padded row
  for (auto& b : h->bufs) {
    hipError_t e = hipMemset(b.p, 0, b.bytes);
    if (e != hipSuccess) {
      ae_status s2 = hip_fail(h, e, "hipMemset");
      ae_destroy(h);
      return s2;
    }
  }
  hipError_t e = hipSuccess;
  if (h->Dc > 0) e = launch_pos_table(h->Pmax + 1, h->dh, cfg->rope_theta, h->pos_cos, h->pos_sin, nullptr);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    ae_destroy(h);
    return AE_ERR_HIP;
  }
  *out = h;
  return AE_OK;
}

ae_status ae_load_weights(ae_handle* h, const ae_tensor_view* w, int n, void* stream) {
  if (!h) return AE_ERR_INVALID_ARGUMENT;
  if (!w || n < 0) return fail(h, AE_ERR_INVALID_ARGUMENT, "null weight list");
  const std::vector<WeightSpec> specs = weight_specs(h);
  std::map<std::string, const ae_tensor_view*> by_name;
  for (int i = 0; i < n; ++i) {
    if (!w[i].name) return fail(h, AE_ERR_INVALID_ARGUMENT, "weight with null name");
    if (by_name.count(w[i].name))
      return fail(h, AE_ERR_INVALID_ARGUMENT, std::string("duplicate weight ") + w[i].name);
    by_name[w[i].name] = &w[i];
  }
  for (const auto& kv : by_name) {
    bool known = false;
    for (const auto& s : specs) known |= s.name == kv.first;
    if (!known) return fail(h, AE_ERR_INVALID_ARGUMENT, "unknown weight " + kv.first);
  }
  for (const auto& s : specs) {
    auto it = by_name.find(s.name);
    if (it == by_name.end()) return fail(h, AE_ERR_INVALID_ARGUMENT, "missing weight " + s.name);
    const ae_tensor_view* v = it->second;
    if (!v->data) return fail(h, AE_ERR_INVALID_ARGUMENT, "null data for " + s.name);
    if (v->dtype != h->cfg.act_dtype)
      return fail(h, AE_ERR_INVALID_ARGUMENT, "dtype of " + s.name + " differs from act_dtype");
    bool ok = v->ndim == static_cast<int>(s.shape.size());
    for (size_t i = 0; ok && i < s.shape.size(); ++i) ok = v->shape[i] == s.shape[i];
    if (!ok)
      return fail(h, AE_ERR_SHAPE_MISMATCH,
                  s.name + " has shape " + shape_str(v->shape, v->ndim > 4 ? 4 : (v->ndim < 0 ? 0 : v->ndim)) +
                      ", expected " + shape_str(s.shape.data(), static_cast<int>(s.shape.size())));
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t es = h->esz;
  const size_t D = h->D;
  auto get = [&](const std::string& nm) { return by_name[nm]->data; };
  auto cp = [&](void* dst, const std::string& nm, size_t bytes) {
    return hipMemcpyAsync(dst, get(nm), bytes, hipMemcpyDeviceToDevice, st);
  };
  // (captured graphs stay valid: they read the packed buffers by address,
  // and the time-path table is rebuilt on the next call)
  h->weights_loaded = false;
  h->table_steps = -1;
  AE_HIP(h, cp(h->tw1, "time_mlp.1.w", D * D * es));
  AE_HIP(h, cp(h->tb1, "time_mlp.1.b", D * es));
  AE_HIP(h, cp(h->tw2, "time_mlp.2.w", D * D * es));
  AE_HIP(h, cp(h->tb2, "time_mlp.2.b", D * es));
  AE_HIP(h, cp(h->fmod_w, "final_mod.w", D * 2 * D * es));
  AE_HIP(h, cp(h->fmod_b, "final_mod.b", 2 * D * es));
  AE_HIP(h, launch_to_f32(h->dt, get("action_in.w"), h->w_in, static_cast<size_t>(h->A) * D, 0, st));
  AE_HIP(h, launch_to_f32(h->dt, get("action_in.b"), h->b_in, D, 0, st));
  AE_HIP(h, launch_to_f32(h->dt, get("action_out.w"), h->w_out, static_cast<size_t>(h->A) * D, h->A, st));
  AE_HIP(h, launch_to_f32(h->dt, get("action_out.b"), h->b_out, h->A, 0, st));
  {
    const int ks = kstep_of(h->dt);
    AE_HIP(h, launch_pack(h->dt, PACK_PLAIN, get("action_in.w"), nullptr, nullptr, h->a_frags * ks, h->D,
                          h->D, 0, 0, h->Hq, h->Hkv, h->dh, h->win_p, st, h->A, h->D));
    AE_HIP(h, launch_pack(h->dt, PACK_PLAIN, get("action_out.w"), nullptr, nullptr, h->D, 16 * h->a_blocks,
                          h->A, 0, 0, h->Hq, h->Hkv, h->dh, h->wout_p, st, h->D, h->A));
  }
  if (h->fp8) {
    // per-tensor amax of q, k, v, gate, up, down -> (448 / amax, amax / 448)
    AE_HIP(h, hipMemsetAsync(h->wamax, 0, static_cast<size_t>(h->L) * 6 * 4, st));
    const char* names[6] = {"q", "k", "v", "gate", "up", "down"};
    const size_t sizes[6] = {D * h->qdim, D * h->kvdim, D * h->kvdim, D * h->F, D * h->F,
                             static_cast<size_t>(h->F) * D};
    for (int l = 0; l < h->L; ++l)
      for (int i = 0; i < 6; ++i)
        AE_HIP(h, launch_weight_amax(static_cast<const uint16_t*>(get("layers." + std::to_string(l) + "." + names[i])),
                                     sizes[i], h->wamax + 6 * l + i, st));
    AE_HIP(h, launch_fp8_scales(h->wamax, h->L * 6, h->wmul, h->wsc, st));
  }
  for (int l = 0; l < h->L && h->Dc > 0; ++l) {
    // [ctx_k | ctx_v] as the QKV packing with no query heads: RoPE pairs of K together
    const std::string p = "layers." + std::to_string(l) + ".";
    AE_HIP(h, launch_pack(h->dt, PACK_QKV, nullptr, get(p + "ctx_k"), get(p + "ctx_v"), h->Dc, 2 * h->kvdim,
                          0, h->kvdim, h->kvdim, 0, h->Hkv, h->dh, h->wctx + l * h->sctx, st));
  }
  if (h->Sd > 0) {
    AE_HIP(h, cp(h->st_w, "state_in.w", static_cast<size_t>(h->Sd) * h->Dc * 2));
    AE_HIP(h, cp(h->st_b, "state_in.b", static_cast<size_t>(h->Dc) * 2));
  }
  for (int l = 0; l < h->L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    const size_t NM = static_cast<size_t>(h->nmod) * D;
    AE_HIP(h, cp(static_cast<char*>(h->mod_w) + l * D * NM * es, p + "mod.w", D * NM * es));
    AE_HIP(h, cp(static_cast<char*>(h->mod_b) + l * NM * es, p + "mod.b", NM * es));
    if (h->dit) {  // q2 in the QKV packing with no K/V heads (its RoPE pairs together)
      AE_HIP(h, launch_pack(h->dt, PACK_QKV, get(p + "q2"), nullptr, nullptr, h->D, h->qdim, h->qdim, 0, 0,
                            h->Hq, 0, h->dh, h->wq2 + l * h->sq2, st));
      AE_HIP(h, launch_pack(h->dt, PACK_PLAIN, get(p + "o2"), nullptr, nullptr, h->qdim, h->D, h->D, 0,
                            0, h->Hq, h->Hkv, h->dh, h->wo2 + l * h->so, st));
    }
    if (!h->fp8o)
      AE_HIP(h, launch_pack(h->dt, PACK_PLAIN, get(p + "o"), nullptr, nullptr, h->qdim, h->D, h->D, 0,
                            0, h->Hq, h->Hkv, h->dh, h->wo + l * h->so, st));
    auto b16 = [&](const std::string& nm) { return static_cast<const uint16_t*>(get(nm)); };
    if (h->rowwise) {
      // a scale per output column of every tensor: multipliers for the
      // packing, and the scales in packed column order for the epilogues
      const int F = h->F, Dm = h->D, qd = h->qdim, kd = h->kvdim;
      float* cm = h->cmul;
      float* cs = h->csc;
      const size_t oq = 0, ok = qd, ov = ok + kd, og = ov + kd, ou = og + F, od = ou + F, oo = od + Dm;
      AE_HIP(h, launch_fp8_col_scales(b16(p + "q"), Dm, qd, qd, cm + oq, cs + oq, st));
      AE_HIP(h, launch_fp8_col_scales(b16(p + "k"), Dm, kd, kd, cm + ok, cs + ok, st));
      AE_HIP(h, launch_fp8_col_scales(b16(p + "v"), Dm, kd, kd, cm + ov, cs + ov, st));
      AE_HIP(h, launch_fp8_col_scales(b16(p + "gate"), Dm, F, F, cm + og, cs + og, st));
      AE_HIP(h, launch_fp8_col_scales(b16(p + "up"), Dm, F, F, cm + ou, cs + ou, st));
      AE_HIP(h, launch_fp8_col_scales(b16(p + "down"), F, Dm, Dm, cm + od, cs + od, st));
      float* sw = h->swc + l * h->swc_layer;
      AE_HIP(h, launch_pack_fp8(PACK_QKV, b16(p + "q"), b16(p + "k"), b16(p + "v"), Dm, h->qkv_n, qd, kd, kd,
                                h->Hq, h->Hkv, h->dh, h->wmul, h->wqkv + l * h->sqkv, st, cm + oq, cm + ok,
                                cm + ov));
      AE_HIP(h, launch_pack_col_scales(PACK_QKV, cs + oq, cs + ok, cs + ov, h->qkv_n, h->Hq, h->Hkv, h->dh, sw, st));
      AE_HIP(h, launch_pack_fp8(PACK_GU, b16(p + "gate"), b16(p + "up"), nullptr, Dm, 2 * F, F, F, 0, h->Hq,
                                h->Hkv, h->dh, h->wmul, h->wgu + l * h->sgu, st, cm + og, cm + ou));
      AE_HIP(h, launch_pack_col_scales(PACK_GU, cs + og, cs + ou, nullptr, 2 * F, h->Hq, h->Hkv, h->dh,
                                       sw + h->qkv_n, st));
      AE_HIP(h, launch_pack_fp8(PACK_PLAIN, b16(p + "down"), nullptr, nullptr, F, Dm, Dm, 0, 0, h->Hq, h->Hkv,
                                h->dh, h->wmul, h->wd + l * h->sd, st, cm + od));
      AE_HIP(h, launch_pack_col_scales(PACK_PLAIN, cs + od, nullptr, nullptr, Dm, h->Hq, h->Hkv, h->dh,
                                       sw + h->qkv_n + 2 * F, st));
      if (h->fp8o) {
        AE_HIP(h, launch_fp8_col_scales(b16(p + "o"), qd, Dm, Dm, cm + oo, cs + oo, st));
        AE_HIP(h, launch_pack_fp8(PACK_PLAIN, b16(p + "o"), nullptr, nullptr, qd, Dm, Dm, 0, 0, h->Hq, h->Hkv,
                                  h->dh, h->wmul, h->wo + l * h->so, st, cm + oo));
        AE_HIP(h, launch_pack_col_scales(PACK_PLAIN, cs + oo, nullptr, nullptr, Dm, h->Hq, h->Hkv, h->dh,
                                         sw + h->qkv_n + 2 * F + Dm, st));
      }
      continue;
    }
    if (h->fp8) {
      AE_HIP(h, launch_pack_fp8(PACK_QKV, b16(p + "q"), b16(p + "k"), b16(p + "v"), h->D, h->qkv_n,
                                h->qdim, h->kvdim, h->kvdim, h->Hq, h->Hkv, h->dh, h->wmul + 6 * l,
                                h->wqkv + l * h->sqkv, st));
      AE_HIP(h, launch_pack_fp8(PACK_GU, b16(p + "gate"), b16(p + "up"), nullptr, h->D, 2 * h->F, h->F,
                                h->F, 0, h->Hq, h->Hkv, h->dh, h->wmul + 6 * l + 3, h->wgu + l * h->sgu, st));
      AE_HIP(h, launch_pack_fp8(PACK_PLAIN, b16(p + "down"), nullptr, nullptr, h->F, h->D, h->D, 0, 0,
                                h->Hq, h->Hkv, h->dh, h->wmul + 6 * l + 5, h->wd + l * h->sd, st));
      continue;
    }
    AE_HIP(h, launch_pack(h->dt, PACK_QKV, get(p + "q"), get(p + "k"), get(p + "v"), h->D, h->qkv_n,
                          h->qdim, h->kvdim, h->kvdim, h->Hq, h->Hkv, h->dh, h->wqkv + l * h->sqkv, st));
    AE_HIP(h, launch_pack(h->dt, PACK_GU, get(p + "gate"), get(p + "up"), nullptr, h->D, 2 * h->F,
                          h->F, h->F, 0, h->Hq, h->Hkv, h->dh, h->wgu + l * h->sgu, st));
    AE_HIP(h, launch_pack(h->dt, PACK_PLAIN, get(p + "down"), nullptr, nullptr, h->F, h->D, h->D, 0,
                          0, h->Hq, h->Hkv, h->dh, h->wd + l * h->sd, st));
  }
  h->weights_loaded = true;
  return AE_OK;
}

ae_status ae_set_prefix_kv(ae_handle* h, int batch, int prefix_len, const void* K, const void* V,
                           const uint8_t* valid_mask, void* stream) {
  if (!h) return AE_ERR_INVALID_ARGUMENT;
  if (batch < 1 || batch > h->Bmax)
    return fail(h, AE_ERR_SHAPE_MISMATCH,
                "batch " + std::to_string(batch) + " outside [1, " + std::to_string(h->Bmax) + "]");
  if (prefix_len < 0 || prefix_len > h->Pmax)
    return fail(h, AE_ERR_SHAPE_MISMATCH,
                "prefix_len " + std::to_string(prefix_len) + " outside [0, " + std::to_string(h->Pmax) + "]");
  if (prefix_len > 0 && (!K || !V || !valid_mask))
    return fail(h, AE_ERR_INVALID_ARGUMENT, "null K, V or valid_mask");
  if (prefix_len > 0 && (reinterpret_cast<uintptr_t>(K) % 16 || reinterpret_cast<uintptr_t>(V) % 16))
    return fail(h, AE_ERR_INVALID_ARGUMENT, "K and V must be 16-byte aligned (the copy moves 16-byte pieces)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the smallest bucket holding the prefix: its rows past prefix_len count
  // as padding (mask 0), and the calls plan their key splits for it
  const int span = pick_bucket(h->buckets, prefix_len, h->Pmax);
  h->prefix_batch = -1;  // (a failed launch leaves no usable prefix)
  AE_HIP(h, launch_prefix_scan(valid_mask, batch, prefix_len, h->comp_idx, h->n_valid, h->T, h->dh,
                               h->cfg.rope_theta, h->rope_cos, h->rope_sin, st, 0, h->src_of));
  AE_HIP(h, launch_prefix_copy(h->dt, K, V, h->src_of, h->n_valid, h->T, h->L, batch, prefix_len,
                               h->Hkv, h->dh, h->Bmax, h->S_max, h->kcache, h->vtcache, st));
  h->prefix_batch = batch;
  h->span = span;
  h->stats.prefix_sets++;
  return AE_OK;
}

ae_status ae_prepare_prefix(ae_handle* h, int batch, int prefix_len, const void* hidden,
                            const uint8_t* valid_mask, const float* state, void* stream) {
  if (!h) return AE_ERR_INVALID_ARGUMENT;
  if (h->Dc == 0) return fail(h, AE_ERR_UNSUPPORTED, "context_width is 0: no context projection");
  if (state && h->Sd == 0) return fail(h, AE_ERR_UNSUPPORTED, "state given but state_dim is 0");
  const int extra = state ? 1 : 0;
  if (batch < 1 || batch > h->Bmax)
    return fail(h, AE_ERR_SHAPE_MISMATCH,
                "batch " + std::to_string(batch) + " outside [1, " + std::to_string(h->Bmax) + "]");
  if (prefix_len < 0 || prefix_len + extra > h->Pmax)
    return fail(h, AE_ERR_SHAPE_MISMATCH,
                "prefix_len " + std::to_string(prefix_len) + (extra ? " + the state row" : "") + " outside [0, " +
                    std::to_string(h->Pmax) + "]");
  if (prefix_len > 0 && (!hidden || !valid_mask)) return fail(h, AE_ERR_INVALID_ARGUMENT, "null hidden or valid_mask");
  if (!h->weights_loaded) return fail(h, AE_ERR_NOT_READY, "weights not loaded");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int span = pick_bucket(h->buckets, prefix_len + extra, h->Pmax);
  const size_t kv_layer = static_cast<size_t>(h->Bmax) * h->Hkv * h->S_max * h->dh * h->esz;
  h->prefix_batch = -1;  // (a failed launch leaves no usable prefix)
  // counts (the state row included), compaction index, action RoPE tables
  AE_HIP(h, launch_prefix_scan(valid_mask, batch, prefix_len, h->comp_idx, h->n_valid, h->T, h->dh,
                               h->cfg.rope_theta, h->rope_cos, h->rope_sin, st, extra));
  if (state)
    AE_HIP(h, launch_state_prep(state, batch, h->Sd, h->st_w, h->st_b, h->Dc, h->n_valid, h->st_h, h->st_key, st));
  // one product per layer: [K | V] of every context row, K rotated at the
  // row's count position, visible rows scattered to their keys
  // every layer in one launch (their packed weights are consecutive); layer
  // l's A rows start a_layer_bytes after layer 0's (0: the same rows for all)
  auto project = [&](const void* A, size_t a_layer_bytes, int rows, int rows_per_req, const int* keys) -> ae_status {
    const int N = h->L * 2 * h->kvdim;
    const TGemmPlan g = plan_tgemm(rows, N, h->Dc, tgemm_kc(OP_BF16), kTargetBlocks);
    TGemmArgs a = base_tgemm(h, h->own, g, rows, N, h->Dc);
    a.ctx_layer_cols = 2 * h->kvdim;
    a.ctx_layer_elems = kv_layer / h->esz;
    a.a_layer_bytes = a_layer_bytes;
    a.A = A;
    a.lda_bytes = static_cast<size_t>(h->Dc) * 2;
    a.W = h->wctx;
    a.kcache = h->kcache;
    a.vtcache = h->vtcache;
    a.n_valid = h->n_valid;
    a.T = rows_per_req; a.Hq = 0; a.Hkv = h->Hkv; a.dh = h->dh; a.S_max = h->S_max;
    a.key_map = keys;
    a.pos_cos = h->pos_cos;
    a.pos_sin = h->pos_sin;
    const hipError_t e = launch_tgemm(OP_BF16, EPI_QKV, a, g.blocks, st);
    return e == hipSuccess ? AE_OK : hip_fail(h, e, "launch_tgemm (context)");
  };
  if (prefix_len > 0) {  // hidden [L][batch][prefix_len][Dc]
    const ae_status r = project(hidden, static_cast<size_t>(batch) * prefix_len * h->Dc * 2, batch * prefix_len,
                                prefix_len, h->comp_idx);
    if (r != AE_OK) return r;
  }
  if (state) {  // the state row is the same input to every layer
    const ae_status r = project(h->st_h, 0, batch, 1, h->st_key);
    if (r != AE_OK) return r;
  }
  // finite values in the rest of each request's last key block (no rows copied)
  AE_HIP(h, launch_prefix_copy(h->dt, nullptr, nullptr, h->src_of, h->n_valid, h->T, h->L, batch, 0, h->Hkv,
                               h->dh, h->Bmax, h->S_max, h->kcache, h->vtcache, st));
  h->prefix_batch = batch;
  h->span = span;
  h->stats.prefix_sets++;
  return AE_OK;
}

ae_status ae_set_prefix_buckets(ae_handle* h, const int* lengths, int n) {
  if (!h) return AE_ERR_INVALID_ARGUMENT;
  if (!valid_buckets(lengths, n, h->Pmax, kMaxBuckets))
    return fail(h, AE_ERR_INVALID_ARGUMENT,
                "prefix buckets must be at most " + std::to_string(kMaxBuckets) +
                    " strictly increasing lengths in [1, max_prefix_len = " + std::to_string(h->Pmax) + "]");
  h->buckets.assign(lengths, lengths + n);
  return AE_OK;
}

ae_status ae_denoise(ae_handle* h, const float* noise, int batch, int steps, float* actions_out,
                     void* stream) {
  if (!h) return AE_ERR_INVALID_ARGUMENT;
  {
    const ae_status c = check_denoise(h, noise, batch, steps, actions_out);
    if (c != AE_OK) return c;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t xbytes = static_cast<size_t>(batch) * h->T * h->A * 4;
  {
    const ae_status t = ensure_tpath(h, steps, st);
    if (t != AE_OK) return t;
  }
  AE_HIP(h, hipMemcpyAsync(h->x, noise, xbytes, hipMemcpyDeviceToDevice, st));
  const bool persist = use_persist(h, batch);
  auto enqueue = [&](hipStream_t s) -> ae_status {
    if (persist) {
      const PersistArgs a = persist_args(h, h->own, batch, steps);
      const hipError_t e = launch_persist(h->dt, a, s);
      return e == hipSuccess ? AE_OK : hip_fail(h, e, "launch_persist");
    }
    return enqueue_loop(h, h->own, batch, steps, s);
  };
  bool ran = false;
  reap_retired(h);
  if (h->graphs.capacity() > 0 && !(persist && !h->persist_graph)) {
    const CallKey key{batch, steps, h->span};
    GraphEntry* ge = h->graphs.find(key);
    if (ge) {
      h->stats.graph_hits++;
    } else {
      h->stats.graph_misses++;
      if (h->graphs.size() < h->graphs.capacity() || h->cfg.graph_cache_evict) {
        AE_HIP(h, hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeRelaxed));
        ae_status s = enqueue(h->cap_stream);
        hipGraph_t graph = nullptr;
        hipError_t e = hipStreamEndCapture(h->cap_stream, &graph);
        GraphEntry ne;
        if (s == AE_OK && e == hipSuccess) e = hipGraphGetNodes(graph, nullptr, &ne.nodes);
        if (s == AE_OK && e == hipSuccess) e = hipGraphInstantiate(&ne.exec, graph, nullptr, nullptr, 0);
        if (graph) (void)hipGraphDestroy(graph);
        if (s == AE_OK && e == hipSuccess) e = hipEventCreateWithFlags(&ne.done, hipEventDisableTiming);
        if (s != AE_OK || e != hipSuccess) {
          (void)hipGetLastError();
          destroy_entry(ne);
          if (!persist) return s != AE_OK ? s : hip_fail(h, e, "graph capture");
          h->persist_graph = false;  // cooperative launches not capturable here: launch directly
        } else {
          GraphEntry old;
          if (h->graphs.insert(key, ne, &old)) {  // the least recently used graph made room
            h->retired.push_back(old);
            h->stats.graph_evictions++;
          }
          ge = h->graphs.find(key);
          h->stats.graph_captures++;
        }
      }
    }
    if (ge) {
      AE_HIP(h, hipGraphLaunch(ge->exec, st));
      AE_HIP(h, hipEventRecord(ge->done, st));
      h->stats.graph_replays++;
      h->stats.graph_nodes = static_cast<long long>(ge->nodes);
      ran = true;
    }
  }
  if (!ran) {
    ae_status s = enqueue(st);
    if (s != AE_OK) return s;
    h->stats.eager_runs++;
    h->stats.graph_nodes = 0;
  }
  if (persist) h->stats.persistent_calls++;
  AE_HIP(h, hipMemcpyAsync(actions_out, h->x, xbytes, hipMemcpyDeviceToDevice, st));
  h->stats.denoise_calls++;
  return AE_OK;
}

ae_status ae_denoise_static(ae_handle* h, const float* noise, int batch, int steps, float* actions_out,
                            void* stream) {
  if (!h) return AE_ERR_INVALID_ARGUMENT;
  {
    const ae_status c = check_denoise(h, noise, batch, steps, actions_out);
    if (c != AE_OK) return c;
  }
  const bool persist = use_persist(h, batch);
  const ScratchNeed need = scratch_need(h, batch, h->span, persist, false);
  ScratchSet sc;
  const size_t bytes = carve(nullptr, need, &sc);
  if (bytes > kStaticScratchBytes)
    return fail(h, AE_ERR_UNSUPPORTED,
                "this call needs " + std::to_string(bytes) + " bytes of scratch; the static scratch holds " +
                    std::to_string(kStaticScratchBytes) + " (ae_denoise has no such limit)");
  char* base = static_cast<char*>(static_scratch(h->device));
  if (!base) return fail(h, AE_ERR_HIP, "the static scratch has no address on this device");
  carve(base, need, &sc);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t xbytes = static_cast<size_t>(batch) * h->T * h->A * 4;
  {
    const ae_status t = ensure_tpath(h, steps, st);
    if (t != AE_OK) return t;
  }
  AE_HIP(h, hipMemcpyAsync(h->x, noise, xbytes, hipMemcpyDeviceToDevice, st));
  if (persist) {
    // (the counter fill before the launch zeroes the flags and counters)
    const PersistArgs a = persist_args(h, sc, batch, steps);
    AE_HIP(h, launch_persist(h->dt, a, st));
    h->stats.persistent_calls++;
  } else {
    // the split counters start at zero (another call may have left other
    // data in this part of the shared memory)
    AE_HIP(h, launch_zero_ints(sc.gcnt, need.gcn, st));
    AE_HIP(h, launch_zero_ints(sc.acnt, need.acn, st));
    const ae_status e = enqueue_loop(h, sc, batch, steps, st);
    if (e != AE_OK) return e;
  }
  AE_HIP(h, hipMemcpyAsync(actions_out, h->x, xbytes, hipMemcpyDeviceToDevice, st));
  h->stats.eager_runs++;
  h->stats.graph_nodes = 0;
  h->stats.denoise_calls++;
  return AE_OK;
}

}  // extern "C"
