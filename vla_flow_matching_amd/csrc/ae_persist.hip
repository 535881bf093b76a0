// The whole denoise call as ONE persistent, cooperatively launched kernel for
// the small-batch regime (batch * T <= 64 rows: one GEMM row tile).
//
// At batch 1 every projection is a skinny GEMM whose weights are streamed
// once per step (MolmoBot PR Part 2: only the action queries and the
// timestep change between flow steps), so the loop is bound by HBM and by
// the dependency chain between phases, not by arithmetic.  Separate kernels
// would pay a launch, a ramp-up and a tail per phase (5 per layer); here every
// workgroup stays resident for the whole call and walks the same phase list:
//
//   IN                      h = x W_in + b_in                (row tiles)
//   per step, per layer:
//     Q   adaRMS(h) . W_qkv -> RoPE -> q, K/V-cache rows    (split-K)
//     A   masked GQA attention over [prefix | actions]      (split-KV)
//     O   h += gate_a * (o . W_o)                           (split-K)
//     G   act = gelu(adaRMS(h) . W_g) * (adaRMS(h) . W_u)   (split-K)
//     D   h += gate_m * (act . W_d)                         (split-K)
//   OUT+IN  v = adaRMS_f(h) W_out + b_out; x += dt v; next h (row tiles)
//
// Latency, not bandwidth, is what the exchange between phases costs, so the
// code keeps every chain of dependent memory round trips short:
//  * phases are separated by a flag barrier: each workgroup publishes its own
//    generation word and a waiting wave reads all words in one round;
//  * before waiting, a workgroup issues the weight loads of its next task
//    into registers, so the HBM stream runs through the synchronisation;
//  * split-K reductions are distributed: every workgroup of a split group
//    publishes its partial tile as (value, generation) packets, one 16-byte
//    store per two values, then reduces only its own slice of rows: it reads
//    that slice of every member's partial until all packets carry the
//    phase's generation (no separate counter round trip), sums in member
//    order (bitwise reproducible) and applies the epilogue.  Attention's key
//    splits join on a per-item counter instead and merge the same way.
//  * activations that cross workgroups use device-coherent 16-byte accesses,
//    issued together and consumed afterwards; weights, the prefix K/V and the
//    time-path tables are read-only in this kernel and use cached loads.
// Counters only grow during a launch (targets are multiples of the split
// count); a fill kernel zeroes them and the barrier words before it and
// advances the generation base past every generation the previous launch
// can have written, so stale packets never match.
// Every wait is bounded: after ~0.2 s a device error flag is raised and the
// kernel drains without waiting again.
#include "ae_device.h"
#include "ae_kernels.h"

namespace ae {

namespace {

constexpr int kThreads = 256;
constexpr int kKpw = 4;  // max k-fragments per wave per GEMM task (weights held in registers)
constexpr int kMaxG = 512;
constexpr long kSpinLimit = 400000;
constexpr int kTileF = kTileM * kTileN;  // floats of one partial tile

// The kernel's arguments, read in place from the kernarg segment.  Every
// phase takes a fresh copy of the segment pointer (laundered through an
// empty asm), so the compiler reloads the fields a phase needs with scalar
// loads at its start instead of holding every argument live in registers
// across the whole call.
using KArgs = const __attribute__((address_space(4))) PersistArgs;

__device__ __forceinline__ PGemm plan_of(const __attribute__((address_space(4))) PGemm& g) {
  PGemm r;
  r.n_tiles = g.n_tiles;
  r.k_frags = g.k_frags;
  r.ksplit = g.ksplit;
  r.nb = g.nb;
  return r;
}

__device__ __forceinline__ KArgs& kargs() {
  KArgs* a = (KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(a));
  return *a;
}

__device__ __forceinline__ int ld_flag(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool dev_error(KArgs& p) { return ld_flag(p.err) != 0; }

__device__ __forceinline__ void raise_error(KArgs& p) {
  __hip_atomic_store(p.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void bar_arrive(KArgs& p, int gen) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(p.flags + blockIdx.x, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All workgroups have arrived at generation `gen`.  Wave 0 polls every
// word, and the device error flag, in one round of loads per poll (the flag
// rides along, so a wait costs no extra round trip); it gives up once the
// flag is set or after kSpinLimit polls.
__device__ __forceinline__ void bar_wait(KArgs& p, int gen) {
  if (threadIdx.x < kWave) {
    const Coh cf(p.flags), ce(p.err);
    constexpr int kPer = kMaxG / kWave;
    long spins = 0;
    for (;;) {
      int v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        v[j] = static_cast<int>(cf.ld4(4u * min(static_cast<int>(threadIdx.x) + j * kWave, p.G - 1)));
      const int err = static_cast<int>(ce.ld4(0));
      int ok = 1;
#pragma unroll
      for (int j = 0; j < kPer; ++j) ok &= v[j] >= gen;
      if (__all(ok) || err != 0) break;
      if (++spins > kSpinLimit) {
        if (threadIdx.x == 0) raise_error(p);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Count this workgroup into a split group and wait until `target` members
// have (thread 0 spins; the caller has already waited for its own stores).
__device__ __forceinline__ void group_join(KArgs& p, int* counter, int target) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    int v = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    long spins = 0;
    while (v < target) {
      if (++spins > kSpinLimit || ((spins & 255) == 0 && dev_error(p))) {
        raise_error(p);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = ld_flag(counter);
    }
  }
  __syncthreads();
}

// Row slice of split member s out of n over `rows` rows.
__device__ __forceinline__ void row_slice(int s, int n, int rows, int& r0, int& r1) {
  r0 = (s * rows) / n;
  r1 = ((s + 1) * rows) / n;
}

// ---------------------------------------------------------------------------
// GEMM phase: one 64-row tile, n-tiles x K splits over workgroups, the K
// range of a task split again over the four waves
// ---------------------------------------------------------------------------

// PRO_ADARMS here: A is the shadow ha = T(h (1 + scale)) of the adaRMS
// input, and the norm finishes after the product, per output element:
//   adaRMS(h) W = r_row * (h (1 + scale)) W + shift W,   r_row = 1 / rms(h_row),
// with shift W (`bias`) precomputed per step and layer and r_row from the
// partial sums of squares.  The product can then start as soon as A lands.
struct GemmLayer {
  const uint4* W;
  const void* A;  // T [M][lda]
  int lda;
  const float* bias;  // PRO_ADARMS: shift W, per packed column
  const float* gate;  // EPI_RESID: gate per column
  const float* nsc;   // EPI_RESID: the next norm's scale (writes ha), or null
  void* kc;  // layer's K cache
  void* vt;  // layer's V^T cache
};

// Per-row reciprocal RMS of h from the per-64-column partial sums of
// squares: four threads per row each load every fourth partial (issued early,
// all in flight together), and finish_rms adds them up (two shuffles) into
// s_r.  Rows <= 64, partials <= 64.
__device__ __forceinline__ void issue_rms(KArgs& p, float (&v)[16]) {
  const Coh cs(p.ssq);
  const int row = threadIdx.x / 4, part = threadIdx.x % 4;
  const int rc = min(row, p.M - 1);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int q = min(part + 4 * j, p.ssq_tiles - 1);
    v[j] = cs.ldf(4u * (q * p.ldssq + rc));
  }
}

__device__ __forceinline__ void finish_rms(KArgs& p, const float (&v)[16], float* s_r) {
  const int row = threadIdx.x / 4, part = threadIdx.x % 4;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (part + 4 * j < p.ssq_tiles) acc += v[j];
  acc += xor1_swap(acc);
  acc += xor2_swap(acc);
  if (part == 0 && row < p.M) s_r[row] = 1.0f / sqrtf(acc / static_cast<float>(p.D) + p.eps);
}

// NB: 16-column groups per tile (4: 64 columns; 2: 32 columns, one RoPE or
// gate/up pair, with twice the K fragments per wave in the same registers,
// so a K = 1024 product needs no split).  Lane = tile column in the
// epilogues; with 32 columns lanes 32-63 mirror 0-31 and store nothing.
template <typename T, int PRO, int EPI, int NB = 4>
__device__ __forceinline__ void gemm_phase(KArgs& p, const PGemm g, const GemmLayer& ly,
                                           uint32_t llgen, int gen_wait, char* smem) {
  using MM = Mma<T>;
  constexpr int E = MM::E;
  constexpr int KSTEP = MM::KSTEP;
  constexpr int MT = kTileM / 16;
  constexpr int TN = 16 * NB;       // tile columns
  constexpr int KPW = kKpw * 4 / NB;  // k-fragments per wave (the same weight registers)
  constexpr int kRw = kTileM / 4;  // epilogue rows per wave at most
  constexpr int kRedPer = MT * NB / 4;  // (row tile, column group) blocks each wave sums
  static_assert(NB == 4 || NB == 2, "64- or 32-column tiles");
  static_assert(EPI != EPI_RESID || NB == 4, "the residual epilogues take 64-column tiles");
  auto s_red = reinterpret_cast<f32x4 (*)[MT * NB][kWave]>(smem);
  auto s_y = reinterpret_cast<float (*)[TN + 1]>(smem);
  // row 1/rms (PRO_ADARMS), past the reduction tile
  float* s_r = reinterpret_cast<float*>(smem + 4 * MT * NB * kWave * sizeof(f32x4));

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int rows = p.M;
  const int mtr = (rows + 15) / 16;
  const int n_tasks = g.n_tiles * g.ksplit;
  const Coh coh_a(ly.A);
  bool waited = false;

  for (int t = blockIdx.x; t < n_tasks; t += p.G) {
    const int nt = t / g.ksplit, s = t % g.ksplit;
    const int kf0 = static_cast<int>((static_cast<long long>(s) * g.k_frags) / g.ksplit);
    const int kf1 = static_cast<int>((static_cast<long long>(s + 1) * g.k_frags) / g.ksplit);
    const int cnt = kf1 - kf0 > wave ? (kf1 - kf0 - wave + 3) / 4 : 0;

    // Every load below is issued unconditionally at a clamped, valid address
    // and masked where it is used: a guarded load would make the compiler
    // wait for it on the spot, one round trip per element.

    // weights of this task -> registers, before waiting for the inputs
    uint4 wb[KPW][NB];
    const uint4* Wt = ly.W + static_cast<size_t>(nt) * NB * g.k_frags * kWave + lane;
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int kf = min(kf0 + wave + 4 * c, g.k_frags - 1);
#pragma unroll
      for (int j = 0; j < NB; ++j) wb[c][j] = Wt[(static_cast<size_t>(j) * g.k_frags + kf) * kWave];
    }

    // per-column epilogue constants (they depend only on the step)
    const int lc = lane % TN;  // the lane's tile column
    const float gn = EPI == EPI_RESID ? ly.gate[nt * TN + lc] : 0.0f;
    const float nsc = EPI == EPI_RESID && ly.nsc ? 1.0f + ly.nsc[nt * TN + lc] : 0.0f;
    const float bs = PRO == PRO_ADARMS ? ly.bias[nt * TN + lc] : 0.0f;

    if (!waited) {
      bar_wait(p, gen_wait);
      waited = true;
    }

    // A operand of the task, all in flight together
    const int arow = lane % 16;
    const int acol = E * (lane / 16);
    uint4 araw[KPW][MT];
#pragma unroll
    for (int c = 0; c < KPW; ++c)
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = min(16 * i + arow, rows - 1);
        const int k = min(kf0 + wave + 4 * c, g.k_frags - 1) * KSTEP + acol;
        araw[c][i] = coh_a.ld16(static_cast<uint32_t>(sizeof(T)) * (row * ly.lda + k));
      }
    // the rows' partial sums of squares ride in the same round of loads and
    // are only needed by the epilogue
    float rv[16];
    if (PRO == PRO_ADARMS) issue_rms(p, rv);

    f32x4 acc[MT][NB];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      if (c < cnt) {
        uint4 a[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) a[i] = 16 * i + arow < rows ? araw[c][i] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          if (i < mtr)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = MM::mma(a[i], wb[c][j], acc[i][j]);
      }
    }

    // the four waves' K slices -> one tile in LDS (row-major s_y)
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (i < mtr)
#pragma unroll
        for (int j = 0; j < NB; ++j) s_red[wave][i * NB + j][lane] = acc[i][j];
    __syncthreads();
    // wave w sums blocks w, w + 4, ... (block = row tile * NB + column group)
    f32x4 v[kRedPer];
#pragma unroll
    for (int u = 0; u < kRedPer; ++u) {
      const int blk = wave + 4 * u, i = blk / NB;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < mtr)
#pragma unroll
        for (int w = 0; w < 4; ++w) v[u] += s_red[w][blk][lane];
    }
    if (PRO == PRO_ADARMS) finish_rms(p, rv, s_r);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRedPer; ++u) {
      const int blk = wave + 4 * u, i = blk / NB, j = blk % NB;
      if (i < mtr)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_y[16 * i + 4 * (lane / 16) + e][16 * j + lane % 16] = v[u][e];
    }
    __syncthreads();

    int r0 = 0, r1 = rows;
    if (g.ksplit > 1) row_slice(s, g.ksplit, rows, r0, r1);

    // epilogue inputs of this member's rows (row r0 + wave + 4i, lane =
    // column): loaded only for the wave's own rows, and after the partial
    // is published (outstanding loads would hold up those stores), so they
    // arrive while the group assembles
    float ein[kRw], ecs[kRw], esn[kRw];
    int enb[kRw];
    const int nrw = r1 - r0 > wave ? (r1 - r0 - wave + 3) / 4 : 0;  // the wave's rows
    const int pph = p.dh / 32, half = p.dh / 2;
    int seg = 0, head = 0, jrot = 0;
    const bool hi = (lane & 16) != 0;
    if (EPI == EPI_QKV) {
      const int P = nt * (NB / 2) + lc / 32, pq = p.Hq * pph, pk = p.Hkv * pph;
      int pi;
      if (P < pq) { seg = 0; head = P / pph; pi = P % pph; }
      else if (P < pq + pk) { seg = 1; head = (P - pq) / pph; pi = (P - pq) % pph; }
      else { seg = 2; head = (P - pq - pk) / pph; pi = (P - pq - pk) % pph; }
      jrot = 16 * pi + lane % 16;
    }
#define AE_EPI_LOADS                                                                  \
  if (EPI != EPI_GELU) {                                                              \
    const Coh ch(p.h);                                                                \
    _Pragma("unroll") for (int i = 0; i < kRw; ++i) {                                  \
      if (i < nrw) {                                                                  \
        const int row = r0 + wave + 4 * i;                                            \
        if (EPI == EPI_RESID) {                                                       \
          ein[i] = ch.ldf(4u * (row * p.D + nt * TN + lc));                           \
        } else {                                                                      \
          const int req = row / p.T, tt = row % p.T;                                  \
          const size_t ti2 = (static_cast<size_t>(req) * p.T + tt) * half + jrot;     \
          ecs[i] = p.rope_cos[ti2];                                                   \
          esn[i] = p.rope_sin[ti2];                                                   \
          enb[i] = p.n_valid[req];                                                    \
        }                                                                             \
      }                                                                               \
    }                                                                                 \
  }
    if (g.ksplit == 1) {
      AE_EPI_LOADS
    }
    if (g.ksplit > 1) {
      // Publish the partial as (value, llgen) 8-byte packets, then reduce
      // this member's row slice over all members in order.  Each packet
      // carries its own generation, so the reducer polls the data itself:
      // no store drain, counter or group wait sits between the members'
      // stores and the reduction.
      const Coh cp(reinterpret_cast<uint2*>(p.gpart) + static_cast<size_t>(nt) * g.ksplit * kTileF);
      for (int i = tid; i < rows * (TN / 2); i += kThreads) {
        const int r = i / (TN / 2), c2 = 2 * (i % (TN / 2));
        cp.st16(8u * (s * kTileF + r * TN + c2),
                make_uint4(__float_as_uint(s_y[r][c2]), llgen, __float_as_uint(s_y[r][c2 + 1]), llgen));
      }
      AE_EPI_LOADS
#undef AE_EPI_LOADS
      const int n2 = (r1 - r0) * (TN / 2);  // packet pairs of the slice
      for (int i = tid; i < n2; i += kThreads) {
        const int r = r0 + i / (TN / 2), c2 = 2 * (i % (TN / 2));
        const uint32_t off = 8u * (r * TN + c2);
        float t0 = 0.0f, t1 = 0.0f;
        for (int s0 = 0; s0 < g.ksplit; s0 += 8) {
          uint4 buf[8];
          long spins = 0;
          for (;;) {
            // (only the group's members: the bound is uniform)
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (s0 + j < g.ksplit) buf[j] = cp.ld16(off + 8u * (s0 + j) * kTileF);
            bool ok = true;
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (s0 + j < g.ksplit) ok = ok && buf[j].y == llgen && buf[j].w == llgen;
            if (ok) break;
            if (++spins > kSpinLimit || ((spins & 255) == 0 && dev_error(p))) {
              raise_error(p);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (s0 + j < g.ksplit) {
              t0 += __uint_as_float(buf[j].x);
              t1 += __uint_as_float(buf[j].z);
            }
        }
        s_y[r][c2] = t0;
        s_y[r][c2 + 1] = t1;
      }
      __syncthreads();
    }

    const Coh cvt(ly.vt);
    if (EPI == EPI_RESID) {
      const Coh ch(p.h), cq(p.ssq), cha(p.ha);
#pragma unroll
      for (int i = 0; i < kRw; ++i) {
        const int row = r0 + wave + 4 * i;
        if (row >= r1) continue;
        const float hn = ein[i] + gn * s_y[row][lane];
        ch.stf(4u * (row * p.D + nt * TN + lane), hn);
        if (ly.nsc) {
          const uint32_t off = sizeof(T) * (row * p.D + nt * TN + lane);
          if (sizeof(T) == 2) cha.st2(off, f2bf(hn * nsc));
          else cha.stf(off, hn * nsc);
        }
        const float sq = wave_sum(hn * hn);
        if (lane == 0) cq.stf(4u * (nt * p.ldssq + row), sq);
      }
    } else if (EPI == EPI_GELU) {
      // lanes 32p + jj (jj < 16) hold gate, 32p + 16 + jj the matching up
      const Coh co(p.act);
      for (int row = r0 + wave; row < r1; row += 4) {
        const float y = PRO == PRO_ADARMS ? s_y[row][lc] * s_r[row] + bs : s_y[row][lc];
        const float other = xor16_swap(y);
        if (!hi && lane < TN) {
          const int f = (nt * (NB / 2) + lc / 32) * 16 + lane % 16;
          const float a = gelu_tanh(y) * other;
          if (sizeof(T) == 2) co.st2(2u * (row * p.F + f), f2bf(a));
          else co.stf(4u * (row * p.F + f), a);
        }
      }
    } else if (nt * (NB / 2) >= (p.Hq + p.Hkv) * pph) {
      // EPI_QKV, a V tile (not rotated): V^T rows are head columns, so the
      // member's rows are a run of consecutive keys per column.  Lane
      // (column c / 8, key j = lane % 8) stores column c's key j: one store
      // instruction covers eight columns' runs instead of 64 scattered keys.
      const int pv0 = (p.Hq + p.Hkv) * pph;
      constexpr int NU = TN / 32;  // 32-column passes
      float bsv[NU];
      int colv[NU], bgv[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int vc = (wave + 4 * u) * 8 + lane / 8;  // tile column
        const int P = nt * (NB / 2) + vc / 32 - pv0;
        bsv[u] = PRO == PRO_ADARMS ? ly.bias[nt * TN + vc] : 0.0f;
        colv[u] = ((vc & 16) ? half : 0) + 16 * (P % pph) + vc % 16;
        bgv[u] = P / pph;  // head
      }
      for (int rb = r0; rb < r1; rb += 8) {
        const int row = rb + lane % 8;
        const int rc = min(row, r1 - 1);
        const int req = rc / p.T;
        const int key = p.n_valid[req] + rc % p.T;
        const float rs = PRO == PRO_ADARMS ? s_r[rc] : 1.0f;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int vc = (wave + 4 * u) * 8 + lane / 8;
          const float y = PRO == PRO_ADARMS ? s_y[rc][vc] * rs + bsv[u] : s_y[rc][vc];
          const uint32_t bgi = static_cast<uint32_t>(req * p.Hkv + bgv[u]);
          const uint32_t off =
              sizeof(T) * (bgi * p.S_max * p.dh + static_cast<uint32_t>(KvLayout<T>::v_off(key, colv[u], p.dh)));
          if (row < r1) {
            if (sizeof(T) == 2) cvt.st2(off, f2bf(y));
            else cvt.stf(off, y);
          }
        }
      }
    } else {  // EPI_QKV (q or k): lanes 32p + jj and 32p + 16 + jj are a rotation pair
      const Coh cqo(p.q);
      const int col = (hi ? half : 0) + jrot;  // column within the head
#pragma unroll
      for (int i = 0; i < kRw; ++i) {
        const int row = r0 + wave + 4 * i;
        if (row >= r1) continue;
        const float y = PRO == PRO_ADARMS ? s_y[row][lc] * s_r[row] + bs : s_y[row][lc];
        const float other = xor16_swap(y);
        // (a, b) -> (a cos - b sin, b cos + a sin); v is not rotated
        const float cs = seg < 2 ? ecs[i] : 1.0f, sn = seg < 2 ? esn[i] : 0.0f;
        const float val = hi ? y * cs + other * sn : y * cs - other * sn;
        if (lane >= TN) continue;  // (a 32-column tile: the mirrored half)
        if (seg == 0) {
          const uint32_t off = sizeof(T) * (row * p.qdim + head * p.dh + col);
          if (sizeof(T) == 2) cqo.st2(off, f2bf(val));
          else cqo.stf(off, val);
        } else {
          const int req = row / p.T;
          const int key = enb[i] + row % p.T;
          const size_t bgi = static_cast<size_t>(req) * p.Hkv + head;
          if (seg == 1) {
            const Coh ck(static_cast<T*>(ly.kc) + bgi * p.S_max * p.dh);
            const uint32_t off = sizeof(T) * static_cast<uint32_t>(KvLayout<T>::k_off(key, col, p.dh));
            if (sizeof(T) == 2) ck.st2(off, f2bf(val));
            else ck.stf(off, val);
          } else {
            const Coh cv(static_cast<T*>(ly.vt) + bgi * p.S_max * p.dh);
            const uint32_t off = sizeof(T) * static_cast<uint32_t>(KvLayout<T>::v_off(key, col, p.dh));
            if (sizeof(T) == 2) cv.st2(off, f2bf(val));
            else cv.stf(off, val);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Attention phase: S^T = K Q^T per 16-key block, online softmax per query
// column, O^T = V^T P^T; split over keys, distributed merge.
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ void store4_coh(const Coh& c, uint32_t off, const float* v);
template <>
__device__ __forceinline__ void store4_coh<bf16_t>(const Coh& c, uint32_t off, const float* v) {
  uint2 w;
  w.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
  w.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
  c.st8(off, w);
}
template <>
__device__ __forceinline__ void store4_coh<float>(const Coh& c, uint32_t off, const float* v) {
  c.st16(off, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                         __float_as_uint(v[3])));
}

constexpr int kMergeBatch = 16;  // attention splits merged per round of loads
constexpr int kStageBlk = 2;     // key blocks staged in LDS at a time

// Load one key block's K fragments (S^T = K Q^T operands) and V^T fragments
// (O^T = V^T P^T operands) into LDS; the cache holds them in that fragment
// order (the key-block layout), so each is one contiguous 1 KiB run, and the
// four waves share the loads.  Keys of the last block past k_end are loaded
// as they are: their scores are masked, and the cache is finite there.
// stage_load issues this wave's loads of a block into registers and
// stage_store parks them in LDS; stage_kv does both.
template <typename T, int DH>
constexpr int kv_frags_per_wave() {
  return ((Mma<T>::KSTEP / 16) * (DH / Mma<T>::KSTEP) + DH / 16) / 4;
}

template <typename T, int DH>
__device__ __forceinline__ void stage_load(const T* Kb, const T* Vb, const Coh& ck, const Coh& cv, bool coh,
                                           int kb0, uint4 (&v)[kv_frags_per_wave<T, DH>()]) {
  using MM = Mma<T>;
  constexpr int E = MM::E, KSTEP = MM::KSTEP;
  constexpr int NF = DH / KSTEP, ND = DH / 16, NBLK = KSTEP / 16;
  constexpr int NK = NBLK * NF, FPB = NK + ND;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const uint32_t blk0 = static_cast<uint32_t>(kb0 / KSTEP * KvLayout<T>::block_elems(DH));
#pragma unroll
  for (int j = 0; j < FPB / 4; ++j) {
    const int f = 4 * j + wave;
    const bool isk = j < NK / 4;
    const uint32_t e = blk0 + static_cast<uint32_t>(((isk ? f : f - NK) * kWave + lane) * E);
    if (coh)
      v[j] = (isk ? ck : cv).ld16(sizeof(T) * e);
    else
      v[j] = *reinterpret_cast<const uint4*>((isk ? Kb : Vb) + e);
  }
}

template <typename T, int DH>
__device__ __forceinline__ void stage_store(uint4* dst, const uint4 (&v)[kv_frags_per_wave<T, DH>()]) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < kv_frags_per_wave<T, DH>(); ++j) dst[(4 * j + wave) * kWave + lane] = v[j];
}

template <typename T, int DH>
__device__ __forceinline__ void stage_kv(const T* Kb, const T* Vb, const Coh& ck, const Coh& cv, bool coh,
                                         int kb0, uint4* dst) {
  uint4 v[kv_frags_per_wave<T, DH>()];
  stage_load<T, DH>(Kb, Vb, ck, cv, coh, kb0, v);
  stage_store<T, DH>(dst, v);
}

template <typename T, int DH>
__device__ __forceinline__ void attention_phase(KArgs& p, const void* kc_l, const void* vt_l,
                                                int it, int gen_wait, char* smem) {
  using MM = Mma<T>;
  constexpr int E = MM::E, KSTEP = MM::KSTEP;
  constexpr int NF = DH / KSTEP, ND = DH / 16, NBLK = KSTEP / 16;
  constexpr int PW = ND * kWave * 4 + 32;  // floats of one wave's partial: O^T, then m[16], l[16]

  const int G = p.Hq / p.Hkv;
  const int R = p.T * G;
  const int n_items = p.batch * p.Hkv * p.n_qg;
  const int n_tasks = n_items * p.nsplit;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, grp = lane / 16;
  bool waited = false;

  constexpr int FPB = NBLK * NF + ND;  // 1 KiB fragments per key block: K, then V^T
  static_assert(FPB % 4 == 0 && (NBLK * NF) % 4 == 0, "fragments split evenly over 4 waves");
  // LDS: kStageBlk staged key blocks [FPB][64]
  uint4* s_kv = reinterpret_cast<uint4*>(smem);

  for (int task = blockIdx.x; task < n_tasks; task += p.G) {
    const int item = task / p.nsplit, s = task % p.nsplit;
    const int qg = item % p.n_qg, bg = item / p.n_qg, g = bg % p.Hkv, b = bg / p.Hkv;
    // uniform across the workgroup: keeps the per-block choice between the
    // cached and the coherent K/V path a scalar branch
    const int nv = __builtin_amdgcn_readfirstlane(p.n_valid[b]);
    const int len = nv + p.T;
    // the request's own keys spread evenly over the splits, in whole key
    // blocks (kc_len covers the bucket's largest request)
    const int kc = min(p.kc_len, ((len + p.nsplit - 1) / p.nsplit + KSTEP - 1) / KSTEP * KSTEP);
    const int k_begin = s * kc;
    const int k_end = min(k_begin + kc, len);
    const int n_blk = k_end > k_begin ? (k_end - k_begin + KSTEP - 1) / KSTEP : 0;
    const T* Kb = static_cast<const T*>(kc_l) + static_cast<size_t>(b * p.Hkv + g) * p.S_max * DH;
    const T* Vb = static_cast<const T*>(vt_l) + static_cast<size_t>(b * p.Hkv + g) * p.S_max * DH;
    const Coh ck(Kb), cv(Vb), cq(p.q), co(p.o);

    // Key blocks made only of prefix rows do not depend on this step's QKV
    // phase: waves 1..3 stage their share of the first ones before the
    // barrier wait, so those loads overlap it.  Wave 0 polls the barrier (a
    // wave's loads return in order), so its share follows the wait, in the
    // same round of loads as the queries and the first round's blocks that
    // hold action rows.
    int pre = 0;
    if (!waited) {
      while (pre < n_blk && pre < kStageBlk && k_begin + (pre + 1) * KSTEP <= nv) {
        if (wave != 0)
          stage_kv<T, DH>(Kb, Vb, ck, cv, false, k_begin + pre * KSTEP, s_kv + pre * FPB * kWave);
        ++pre;
      }
      bar_wait(p, gen_wait);
      waited = true;
    }

    const int qr0 = (qg * 4 + wave) * 16;
    const bool active = qr0 < R;
    const int myq = qr0 + lane % 16;
    const bool qvalid = myq < R;
    const int hh = qvalid ? myq / p.T : 0;
    const int tt = qvalid ? myq % p.T : 0;
    // Q^T fragments of this wave's 16 query rows (kept in registers for the
    // key loop) and the first round's key blocks still to stage, all in
    // flight together
    const int nfirst = min(kStageBlk, n_blk);
    uint4 qf[NF];
    {
      const uint32_t qoff = sizeof(T) * ((b * p.T + tt) * p.qdim + (g * G + hh) * DH + E * grp);
#pragma unroll
      for (int kf = 0; kf < NF; ++kf)
        qf[kf] = cq.ld16(qoff + sizeof(T) * kf * KSTEP);  // rows past R: a valid row, unused
      uint4 kv[kStageBlk][kv_frags_per_wave<T, DH>()];
#pragma unroll
      for (int bi = 0; bi < kStageBlk; ++bi) {
        const int kb0 = k_begin + bi * KSTEP;
        if (bi < nfirst && (bi >= pre || wave == 0))
          stage_load<T, DH>(Kb, Vb, ck, cv, kb0 + KSTEP > nv, kb0, kv[bi]);
      }
#pragma unroll
      for (int bi = 0; bi < kStageBlk; ++bi)
        if (bi < nfirst && (bi >= pre || wave == 0)) stage_store<T, DH>(s_kv + bi * FPB * kWave, kv[bi]);
    }
    int staged = nfirst;
    f32x4 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    for (int c0 = 0; c0 < n_blk; c0 += kStageBlk) {
      // stage the rest of this round's blocks (coherently where they hold
      // action rows written by this launch)
      for (int bi = max(staged, c0); bi < min(c0 + kStageBlk, n_blk); ++bi) {
        const int kb0 = k_begin + bi * KSTEP;
        stage_kv<T, DH>(Kb, Vb, ck, cv, kb0 + KSTEP > nv, kb0, s_kv + (bi - c0) * FPB * kWave);
      }
      staged = 0;
      __syncthreads();
      if (active) {
        for (int bi = c0; bi < min(c0 + kStageBlk, n_blk); ++bi) {
          const int kb0 = k_begin + bi * KSTEP;
          const uint4* fr = s_kv + (bi - c0) * FPB * kWave + lane;
          // the block's K and V^T fragments into registers up front, so the
          // LDS reads overlap each other rather than each one the MFMA
          // that consumes it
          uint4 kfr[NBLK * NF], vfr[ND];
#pragma unroll
          for (int f = 0; f < NBLK * NF; ++f) kfr[f] = fr[f * kWave];
#pragma unroll
          for (int d = 0; d < ND; ++d) vfr[d] = fr[(NBLK * NF + d) * kWave];
          f32x4 st[NBLK];
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk) {
            st[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kf = 0; kf < NF; ++kf) st[blk] = MM::mma(kfr[blk * NF + kf], qf[kf], st[blk]);
          }
          float sv[NBLK * 4];
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[blk * 4 + i] = st[blk][i] * p.scale_log2;
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
          cmax = xor32_max(cmax);
          if (!__all(cmax <= m_run + kSoftmaxSlack)) {  // move the reference max
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = exp2_hw(m_run - m_new);
#pragma unroll
            for (int d = 0; d < ND; ++d) acc[d] *= alpha;
            l_run *= alpha;
            m_run = m_new;
          }
          float psum = 0.0f;
#pragma unroll
          for (int i = 0; i < NBLK * 4; ++i) {
            sv[i] = exp2_hw(sv[i] - m_run);
            psum += sv[i];
          }
          psum = xor16_sum(psum);
          psum = xor32_sum(psum);
          l_run += psum;
          const uint4 pf = pack_frag<T>(sv);
#pragma unroll
          for (int d = 0; d < ND; ++d) acc[d] = MM::mma(vfr[d], pf, acc[d]);
        }
      }
      __syncthreads();  // staged blocks are dead before the next round overwrites them
    }
    // acc[d][i] = O^T[dim 16 d + 4 grp + i][query lane % 16] (unnormalised)

    if (p.nsplit == 1) {
      if (active && qvalid) {
        const float inv = 1.0f / l_run;
        const uint32_t obase = sizeof(T) * ((b * p.T + tt) * p.qdim + (g * G + hh) * DH);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          float v[4] = {acc[d][0] * inv, acc[d][1] * inv, acc[d][2] * inv, acc[d][3] * inv};
          store4_coh<T>(co, obase + sizeof(T) * (16 * d + 4 * grp), v);
        }
      }
      continue;
    }

    // publish (O^T, m, l) of this split, join the item's group
    const Coh cpart(p.apart + static_cast<size_t>(item) * p.nsplit * 4 * PW);
    if (active) {
      const uint32_t wbase = 4u * ((s * 4 + wave) * PW);
#pragma unroll
      for (int d = 0; d < ND; ++d)
        cpart.st16(wbase + 16u * (d * kWave + lane),
                   make_uint4(__float_as_uint(acc[d][0]), __float_as_uint(acc[d][1]),
                              __float_as_uint(acc[d][2]), __float_as_uint(acc[d][3])));
      if (grp == 0) {
        cpart.stf(wbase + 4u * (ND * kWave * 4 + lane), m_run);
        cpart.stf(wbase + 4u * (ND * kWave * 4 + 16 + lane), l_run);
      }
    }
    group_join(p, p.acnt + item, p.nsplit * (it + 1));

    // distributed merge: units (wave w of the item, d block) dealt to members
    const int n_units = 4 * ND;
    for (int u = s * 4 + wave; u < n_units; u += 4 * p.nsplit) {
      const int w = u / ND, d = u % ND;
      const int uq0 = (qg * 4 + w) * 16;
      if (uq0 >= R) continue;
      const int q = uq0 + lane % 16;
      // every split's (m, l, O^T piece) requested at once (clamped split
      // index, masked at use), then combined in split order
      float mx = -INFINITY;
      f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
      float lsum = 0.0f;
      for (int s0 = 0; s0 < p.nsplit; s0 += kMergeBatch) {
        float mv[kMergeBatch], lv[kMergeBatch];
        uint4 av[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const uint32_t wb = 4u * ((min(s0 + j, p.nsplit - 1) * 4 + w) * PW);
          mv[j] = cpart.ldf(wb + 4u * (ND * kWave * 4 + lane % 16));
          lv[j] = cpart.ldf(wb + 4u * (ND * kWave * 4 + 16 + lane % 16));
          av[j] = cpart.ld16(wb + 16u * (d * kWave + lane));
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          // an empty split (m = -inf) or a clamped repeat carries no weight
          if (s0 + j >= p.nsplit || mv[j] == -INFINITY) continue;
          const float m_new = fmaxf(mx, mv[j]);
          const float a_old = exp2_hw(mx - m_new), a_new = exp2_hw(mv[j] - m_new);
          lsum = lsum * a_old + lv[j] * a_new;
          o = o * a_old + a_new * f32x4{__uint_as_float(av[j].x), __uint_as_float(av[j].y),
                                        __uint_as_float(av[j].z), __uint_as_float(av[j].w)};
          mx = m_new;
        }
      }
      if (q < R) {
        const int h2 = q / p.T, t2 = q % p.T;
        const float inv = 1.0f / lsum;
        float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        store4_coh<T>(co, sizeof(T) * ((b * p.T + t2) * p.qdim + (g * G + h2) * DH + 16 * d + 4 * grp), v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// OUT + IN phase, one task per 16-row tile:
//   OUT: v = adaRMS(h; scale_f, shift_f) . W_out + b_out, x += dt v
//   IN:  h = x . W_in + b_in, and h's per-64-column row sums of squares
// For bf16 weights, the fp32 operand (u or x) is split into a bf16 high
// part and a bf16 remainder, both multiplied on the MFMA units, which keeps
// these two projections at ~fp32 accuracy (the weights are exact in bf16).
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ void split_frag(const float* v, uint4& hi, uint4& lo);
template <>
__device__ __forceinline__ void split_frag<bf16_t>(const float* v, uint4& hi, uint4& lo) {
  float h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = bf2f(f2bf(v[i]));
    l[i] = v[i] - h[i];
  }
  hi = pack_frag_bf16(h);
  lo = pack_frag_bf16(l);
}
template <>
__device__ __forceinline__ void split_frag<float>(const float* v, uint4& hi, uint4& lo) {
  hi = pack_frag_f32(v);
  lo = make_uint4(0, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void outin_phase(KArgs& p, int step, bool do_out, bool do_in,
                                            int gen_wait, char* smem) {
  using MM = Mma<T>;
  constexpr int E = MM::E, KSTEP = MM::KSTEP;
  constexpr bool kSplit = sizeof(T) == 2;
  constexpr int KPW_OUT = 8;   // h / W_out fragments per wave per chunk
  constexpr int CPW_IN = 16;   // W_in column blocks per wave per chunk
  constexpr int kAF = 32 / KSTEP;  // fragments covering A <= 32
  constexpr int kAB = 2;           // W_out column blocks covering A <= 32
  float* s_x = reinterpret_cast<float*>(smem);        // [16][64]
  float* s_r = s_x + 16 * 64;                         // [16]
  float* s_part = s_r + 16;                           // [ssq_tiles][16]
  float* s_f = s_part + 64 * 16;                      // [2][D]: 1 + scale_f, shift_f
  f32x4* s_red = reinterpret_cast<f32x4*>(s_f + 2 * 4096);  // [4 waves][4 blocks][64]
  float* s_sq = reinterpret_cast<float*>(s_red);             // [16 slots][16 rows] (IN part)
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n_tasks = (p.M + 15) / 16;
  const Coh cx(p.x), ch(p.h), cs(p.ssq), cha(p.ha);
  const int row = lane % 16;
  const int kfr = p.D / KSTEP;       // h / W_out fragments
  const int nb = p.D / 16;           // W_in column blocks
  // the first layer's attention norm scale at the step the new h feeds
  const float* sc_in = p.mod + static_cast<size_t>(do_out ? step + 1 : 0) * p.L * 6 * p.D;
  bool waited = false;

  for (int task = blockIdx.x; task < n_tasks; task += p.G) {
    const int m0 = task * 16;
    const int rows = min(16, p.M - m0);

    // weights of the first chunk of each part, before waiting
    uint4 wo[KPW_OUT][kAB];
#define AE_ISSUE_WOUT(c0)                                                                   \
  _Pragma("unroll") for (int c = 0; c < KPW_OUT; ++c) {                                      \
    const int kf = wave + 4 * ((c0) + c);                                                   \
    _Pragma("unroll") for (int j = 0; j < kAB; ++j) wo[c][j] =                               \
        p.wout_p[(static_cast<size_t>(min(j, p.a_blocks - 1)) * kfr + min(kf, kfr - 1)) * kWave + lane]; \
  }
    uint4 wi[CPW_IN][kAF];
    float bi[CPW_IN], si[CPW_IN];
#define AE_ISSUE_WIN(q0)                                                                    \
  _Pragma("unroll") for (int q = 0; q < CPW_IN; ++q) {                                       \
    const int cb = wave + 4 * ((q0) + q);                                                   \
    bi[q] = p.b_in[16 * min(cb, nb - 1) + lane % 16];                                       \
    si[q] = sc_in[16 * min(cb, nb - 1) + lane % 16];                                        \
    _Pragma("unroll") for (int f = 0; f < kAF; ++f) wi[q][f] =                               \
        p.win_p[(static_cast<size_t>(min(cb, nb - 1)) * p.a_frags + min(f, p.a_frags - 1)) * kWave + lane]; \
  }
    AE_ISSUE_WOUT(0)

    if (!waited) {
      bar_wait(p, gen_wait);
      waited = true;
    }
    // x rows, the rows' partial sums of squares, the final modulation and
    // (OUT) this wave's first h fragments, all in flight together
    float xv[4], pv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + j * kThreads, r = i / 64, a = i % 64;
      // loads at clamped (valid) indices, masked at use
      xv[j] = cx.ldf(4u * ((m0 + min(r, rows - 1)) * p.A + min(a, p.A - 1)));
      const int q = i / 16, r2 = i % 16;
      pv[j] = cs.ldf(4u * (min(q, p.ssq_tiles - 1) * p.ldssq + m0 + min(r2, rows - 1)));
      if (!(r < rows && a < p.A)) xv[j] = 0.0f;
      if (!(do_out && q < p.ssq_tiles && r2 < rows)) pv[j] = 0.0f;
    }
    uint4 hraw[KPW_OUT][E / 4];
#define AE_ISSUE_H(c0)                                                                      \
  _Pragma("unroll") for (int c = 0; c < KPW_OUT; ++c) {                                      \
    const int kf = wave + 4 * ((c0) + c);                                                   \
    const int k = kf * KSTEP + E * (lane / 16);                                             \
    _Pragma("unroll") for (int q = 0; q < E / 4; ++q) hraw[c][q] =                           \
        ch.ld16(4u * ((m0 + min(row, rows - 1)) * p.D + min(k, p.D - E) + 4 * q));          \
  }
    AE_ISSUE_H(0)
    if (do_out) {
      const float* sf = p.fmod + static_cast<size_t>(step) * 2 * p.D;
      for (int i = tid; i < 2 * p.D; i += kThreads) s_f[i] = i < p.D ? 1.0f + sf[i] : sf[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + j * kThreads;
      s_x[i] = xv[j];
      if (i / 16 < p.ssq_tiles) s_part[i] = pv[j];
    }
    __syncthreads();
    if (do_out && tid < rows) {
      float acc = 0.0f;
      for (int q = 0; q < p.ssq_tiles; ++q) acc += s_part[q * 16 + tid];
      s_r[tid] = 1.0f / sqrtf(acc / static_cast<float>(p.D) + p.eps);
    }
    __syncthreads();

    if (do_out) {
      const float rr = row < rows ? s_r[row] : 0.0f;
      f32x4 acc[kAB];
#pragma unroll
      for (int j = 0; j < kAB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; wave + 4 * c0 < kfr; c0 += KPW_OUT) {
        if (c0 > 0) {
          AE_ISSUE_WOUT(c0)
          AE_ISSUE_H(c0)
        }
#pragma unroll
        for (int c = 0; c < KPW_OUT; ++c) {
          const int kf = wave + 4 * (c0 + c);
          if (kf >= kfr) continue;
          const int k = kf * KSTEP + E * (lane / 16);
          float v[E];
#pragma unroll
          for (int q = 0; q < E / 4; ++q) {
            const uint4 hv = hraw[c][q];
            const float hx[4] = {__uint_as_float(hv.x), __uint_as_float(hv.y), __uint_as_float(hv.z),
                                 __uint_as_float(hv.w)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[4 * q + e] = row < rows ? hx[e] * rr * s_f[k + 4 * q + e] + s_f[p.D + k + 4 * q + e] : 0.0f;
          }
          uint4 hi, lo;
          split_frag<T>(v, hi, lo);
#pragma unroll
          for (int j = 0; j < kAB; ++j)
            if (j < p.a_blocks) {
              acc[j] = MM::mma(hi, wo[c][j], acc[j]);
              if (kSplit) acc[j] = MM::mma(lo, wo[c][j], acc[j]);
            }
        }
      }
#pragma unroll
      for (int j = 0; j < kAB; ++j) s_red[(wave * 4 + j) * kWave + lane] = acc[j];
      __syncthreads();
      // x += dt (v + b_out); result row 4*(lane/16)+e, column 16 j + lane % 16
      {
        const int j = tid / kWave, ln = tid % kWave;
        if (j < p.a_blocks) {
          const f32x4 v = s_red[(0 * 4 + j) * kWave + ln] + s_red[(1 * 4 + j) * kWave + ln] +
                          s_red[(2 * 4 + j) * kWave + ln] + s_red[(3 * 4 + j) * kWave + ln];
          const int a = 16 * j + ln % 16;
          const float bo = a < p.A ? p.b_out[a] : 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * (ln / 16) + e;
            if (r < rows && a < p.A) {
              const float xn = s_x[r * 64 + a] + p.dt * (v[e] + bo);
              s_x[r * 64 + a] = xn;
              cx.stf(4u * ((m0 + r) * p.A + a), xn);
            }
          }
        }
      }
      __syncthreads();
    }

    if (do_in) {
      // h[16 x D] = x[16 x A] . W_in + b_in; wave w takes column blocks w + 4q
      AE_ISSUE_WIN(0)
      uint4 ahi[kAF], alo[kAF];
#pragma unroll
      for (int f = 0; f < kAF; ++f) {
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = s_x[row * 64 + f * KSTEP + E * (lane / 16) + e];
        split_frag<T>(v, ahi[f], alo[f]);
      }
      for (int q0 = 0; wave + 4 * q0 < nb; q0 += CPW_IN) {
        if (q0 > 0) {
          AE_ISSUE_WIN(q0)
        }
#pragma unroll
        for (int q = 0; q < CPW_IN; ++q) {
          const int cb = wave + 4 * (q0 + q);
          // 64-column tile cb / 4 is assembled from the four waves' blocks
          float sq[4] = {0.f, 0.f, 0.f, 0.f};
          if (cb < nb) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int f = 0; f < kAF; ++f)
              if (f < p.a_frags) {
                acc = MM::mma(ahi[f], wi[q][f], acc);
                if (kSplit) acc = MM::mma(alo[f], wi[q][f], acc);
              }
            const int n = 16 * cb + lane % 16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * (lane / 16) + e;
              const float hv = acc[e] + bi[q];
              if (r < rows) {
                ch.stf(4u * ((m0 + r) * p.D + n), hv);
                const float ha = hv * (1.0f + si[q]);
                if (sizeof(T) == 2) cha.st2(sizeof(T) * ((m0 + r) * p.D + n), f2bf(ha));
                else cha.stf(sizeof(T) * ((m0 + r) * p.D + n), ha);
                sq[e] = hv * hv;
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) sq[e] = row16_sum(sq[e]);
          if (lane % 16 == 0)
#pragma unroll
            for (int e = 0; e < 4; ++e) s_sq[(q * 4 + wave) * 16 + 4 * (lane / 16) + e] = sq[e];
          __builtin_amdgcn_sched_barrier(0);  // one output block at a time
        }
        __syncthreads();
        // tile (q0 + q): blocks 4 (q0 + q) + w, w = 0..3
        for (int i = tid; i < CPW_IN * 16; i += kThreads) {
          const int q = i / 16, r = i % 16;
          const int tile = q0 + q;
          if (r < rows && 64 * tile < p.D) {
            float t = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) t += s_sq[(q * 4 + w) * 16 + r];
            cs.stf(4u * (tile * p.ldssq + m0 + r), t);
          }
        }
        __syncthreads();
      }
    }
    __syncthreads();
  }
#undef AE_ISSUE_WOUT
#undef AE_ISSUE_WIN
#undef AE_ISSUE_H
}

// LDS of the whole-call kernel: the largest phase's need (GEMM: 64 KiB
// reduction tile + rms / modulation scratch; attention: Q^T fragments and
// kStageBlk staged key blocks).
template <typename T, int DH>
constexpr int smem_bytes() {
  constexpr int gemm = 4 * (kTileM / 16) * (kTileN / 16) * kWave * 16 + 24 * 1024;
  constexpr int nf = DH / Mma<T>::KSTEP, fpb = (Mma<T>::KSTEP / 16) * nf + DH / 16;
  constexpr int attn = kStageBlk * fpb * kWave * 16;
  return gemm > attn ? gemm : attn;
}

template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void persist_kernel(PersistArgs) {
  // gemm: 64 KiB reduction / tile + rms scratch; out/in: smaller
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<T, DH>()];
  // generation base of this launch's split-K packets (set by the counter
  // fill that precedes every launch)
  const uint32_t gbase = __builtin_amdgcn_readfirstlane(kargs().genp[1]);
  int gen = 0;
  outin_phase<T>(kargs(), 0, false, true, 0, smem);  // h from x_0
  bar_arrive(kargs(), ++gen);
  for (int k = 0; k < kargs().n_steps; ++k) {
    for (int l = 0; l < kargs().L; ++l) {
      const int it = k * kargs().L + l;
      {
        KArgs& p = kargs();
        GemmLayer ly;
        ly.kc = static_cast<char*>(p.kcache) + l * p.kv_layer * sizeof(T);
        ly.vt = static_cast<char*>(p.vtcache) + l * p.kv_layer * sizeof(T);
        ly.gate = nullptr;
        ly.nsc = nullptr;
        ly.W = p.wqkv + l * p.sqkv; ly.A = p.ha; ly.lda = p.D; ly.bias = p.bq + static_cast<size_t>(it) * p.qkv_n;
        gemm_phase<T, PRO_ADARMS, EPI_QKV>(p, plan_of(p.pq), ly, gbase + 8 * it + 1, gen, smem);
        bar_arrive(p, ++gen);
      }
      {
        KArgs& p = kargs();
        attention_phase<T, DH>(p, static_cast<char*>(p.kcache) + l * p.kv_layer * sizeof(T),
                               static_cast<char*>(p.vtcache) + l * p.kv_layer * sizeof(T), it, gen, smem);
        bar_arrive(p, ++gen);
      }
      {
        KArgs& p = kargs();
        const float* md = p.mod + static_cast<size_t>(it) * 6 * p.D;
        GemmLayer ly;
        ly.kc = ly.vt = nullptr;
        ly.bias = nullptr;
        ly.W = p.wo + l * p.so; ly.A = p.o; ly.lda = p.qdim; ly.gate = md + 2 * p.D; ly.nsc = md + 3 * p.D;
        gemm_phase<T, PRO_NONE, EPI_RESID>(p, plan_of(p.po), ly, gbase + 8 * it + 2, gen, smem);
        bar_arrive(p, ++gen);
      }
      {
        KArgs& p = kargs();
        GemmLayer ly;
        ly.kc = ly.vt = nullptr;
        ly.gate = ly.nsc = nullptr;
        ly.W = p.wgu + l * p.sgu; ly.A = p.ha; ly.lda = p.D; ly.bias = p.bg + static_cast<size_t>(it) * 2 * p.F;
        const PGemm pg = plan_of(p.pg);
        bool narrow = false;
        if constexpr (sizeof(T) == 2) {
          if (pg.nb == 2) {
            gemm_phase<T, PRO_ADARMS, EPI_GELU, 2>(p, pg, ly, gbase + 8 * it + 3, gen, smem);
            narrow = true;
          }
        }
        if (!narrow) gemm_phase<T, PRO_ADARMS, EPI_GELU>(p, pg, ly, gbase + 8 * it + 3, gen, smem);
        bar_arrive(p, ++gen);
      }
      {
        // the next layer's attention norm scale (the last layer's h goes to
        // the final norm, which reads h itself)
        KArgs& p = kargs();
        const float* md = p.mod + static_cast<size_t>(it) * 6 * p.D;
        GemmLayer ly;
        ly.kc = ly.vt = nullptr;
        ly.bias = nullptr;
        ly.W = p.wd + l * p.sd; ly.A = p.act; ly.lda = p.F; ly.gate = md + 5 * p.D;
        ly.nsc = l + 1 < p.L ? md + 6 * p.D : nullptr;
        gemm_phase<T, PRO_NONE, EPI_RESID>(p, plan_of(p.pd), ly, gbase + 8 * it + 4, gen, smem);
        bar_arrive(p, ++gen);
      }
    }
    outin_phase<T>(kargs(), k, true, k + 1 < kargs().n_steps, gen, smem);
    bar_arrive(kargs(), ++gen);
  }
}

template <typename T, int DH>
hipError_t launch_p(const PersistArgs& a, hipStream_t s) {
  void* args[] = {const_cast<PersistArgs*>(&a)};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(persist_kernel<T, DH>), dim3(a.G),
                                    dim3(kThreads), args, 0, s);
}

template <typename T, int DH>
int occupancy_p() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, persist_kernel<T, DH>, kThreads, 0) != hipSuccess)
    return 0;
  return n;
}

// Zero the barrier flags and split counters, advance the packet generation
// base past every generation the previous launch used, and re-arm the error
// flag.
__global__ void fill_int_kernel(PersistArgs args, uint32_t stride) {
  const int na = args.G;
  const int nb = args.pq.n_tiles + args.po.n_tiles + args.pg.n_tiles + args.pd.n_tiles + args.n_acnt;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < na + nb; i += gridDim.x * blockDim.x) {
    if (i < na) args.flags[i] = 0;
    else args.pcnt[i - na] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // this launch's base is the end of the previous launch's range
    // (genp[0]); the next launch starts past every generation this one can
    // use, whatever either one's layer count
    const uint32_t base = args.genp[0];
    args.genp[1] = base;
    args.genp[0] = base + stride;
    // err[0] is this launch's flag; a flag the previous launch raised is
    // counted into err[1] and cleared, so one timed-out barrier does not
    // disarm the waits of every later launch
    if (args.err[0] != 0) {
      args.err[1] += 1;
      args.err[0] = 0;
    }
  }
}

}  // namespace

int persist_kpw() { return kKpw; }
int persist_max_grid() { return kMaxG; }

int persist_blocks_per_cu(Dt dt, int dh) {
  if (dt == DT_BF16) {
    if (dh == 64) return occupancy_p<bf16_t, 64>();
    if (dh == 128) return occupancy_p<bf16_t, 128>();
    if (dh == 256) return occupancy_p<bf16_t, 256>();
  } else {
    if (dh == 64) return occupancy_p<float, 64>();
    if (dh == 128) return occupancy_p<float, 128>();
    if (dh == 256) return occupancy_p<float, 256>();
  }
  return 0;
}

hipError_t launch_persist(Dt dt, const PersistArgs& a, hipStream_t s) {
  if (a.G < 1 || a.G > kMaxG) return hipErrorInvalidValue;
  const int n_cnt = a.pq.n_tiles + a.po.n_tiles + a.pg.n_tiles + a.pd.n_tiles;
  // a launch takes the next range of generations (8 per layer step), so no
  // two launches ever share one
  const uint32_t stride = 8u * static_cast<uint32_t>(a.n_steps * a.L) + 8u;
  (void)n_cnt;
  hipLaunchKernelGGL(fill_int_kernel, dim3(4), dim3(256), 0, s, a, stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == DT_BF16) {
    if (a.dh == 64) return launch_p<bf16_t, 64>(a, s);
    if (a.dh == 128) return launch_p<bf16_t, 128>(a, s);
    if (a.dh == 256) return launch_p<bf16_t, 256>(a, s);
  } else {
    if (a.dh == 64) return launch_p<float, 64>(a, s);
    if (a.dh == 128) return launch_p<float, 128>(a, s);
    if (a.dh == 256) return launch_p<float, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ae
