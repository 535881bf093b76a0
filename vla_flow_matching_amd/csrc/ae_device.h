// Device-side building blocks shared by the kernels: element types, the
// 16x16 MFMA fragment conventions, conversions and cross-workgroup sync.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ae {

typedef uint16_t bf16_t;  // storage type of bfloat16 values

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Element type traits: storage <-> fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};

// ---------------------------------------------------------------------------
// 16x16 MFMA fragments.
//
// A fragment is 16 bytes per lane.  With E elements per lane (bf16: 8,
// fp32: 4), one fragment covers a 16 x (4E) block: lane l holds row
// (l % 16) and the E consecutive k indices 4E-block-local E*(l/16) .. +E-1.
// The A operand (rows = output rows) and the B operand (rows = output
// columns, i.e. B^T) use the same lane map, so any order in which the
// hardware consumes the E values of a lane is matched on both sides.
// The 16x16 fp32 result: lane l, element i -> row 4*(l/16)+i, column l%16.
// ---------------------------------------------------------------------------

template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int E = 8;      // elements per lane per fragment
  static constexpr int KSTEP = 32; // k covered by one fragment
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int E = 4;
  static constexpr int KSTEP = 16;
  // four 16x16x4 MFMAs, element i of every lane forming k-slice i
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

// ---------------------------------------------------------------------------
// Direct global -> LDS copies.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// One fragment copied from global memory straight into LDS: lane l's 16
// bytes at g + lane16 (= 16 l) land at LDS byte address lds + 16 l; g and
// lds are wave-uniform (scalar registers).  Issued as inline assembly so that
// the compiler neither moves it nor adds waits for it; the caller waits with
// wait_vm before a barrier.
__device__ __forceinline__ void dma_frag(const void* g, uint32_t lds, uint32_t lane16) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(lane16), "s"(g), "s"(lds) : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// A prefetch workgroup (w of nwg, NT threads): its waves stream 1 KiB pieces
// of the ranges src[r] (n4[r] 16-byte words each, r < nr) through PIECES KiB
// of this workgroup's LDS at byte address lds0.  The bytes are dropped; what
// matters is that they sit in the last-level cache when the next kernels
// read them.  Up to PIECES pieces are in flight per wave.
template <int NT, int PIECES>
__device__ __forceinline__ void prefetch_ranges(const uint4* const* src, const int* n4, int nr, int w, int nwg,
                                                uint32_t lds0) {
  const int gw = __builtin_amdgcn_readfirstlane(w * (NT / kWave) + static_cast<int>(threadIdx.x) / kWave);
  const int nw = nwg * (NT / kWave);
  const uint32_t lane16 = 16u * (threadIdx.x % kWave);
  for (int r = 0; r < nr; ++r) {
    const int nf = n4[r] / kWave;
    int cnt = 0;
    for (int f = gw; f < nf; f += nw) {
      dma_frag(src[r] + static_cast<size_t>(f) * kWave, lds0 + static_cast<uint32_t>(cnt % PIECES) * 1024u, lane16);
      if (++cnt % PIECES == 0) wait_vm<0>();
    }
  }
  wait_vm<0>();
}

// ---------------------------------------------------------------------------
// Key-block K / V cache layout.
//
// The keys of one (request, KV head) are stored in blocks of KB = KSTEP keys
// (bf16: 32, fp32: 16), each block in the fragment order the attention
// kernels multiply from, so that one block is one contiguous run per
// operand: the K cache holds NBLK * NF fragments per block (S^T = K Q^T
// A-operands, fragment blk * NF + kf = keys of 16-row tile blk, dims
// kf * KSTEP ..), the V cache ND = dh / 16 fragments (O^T = V^T P^T
// A-operands, fragment fd = dims 16 fd .. 16 fd + 15).
//
// Row r of tile blk is block-local key key_of(blk, r) = E (r / 4) + 4 blk +
// r % 4.  The 16x16 S^T result puts rows 4 g .. 4 g + 3 in lane group g, so
// lane group g ends up with keys E g .. E g + E - 1 in order over the NBLK
// tiles: exactly the k-slice of a P^T fragment, whose V^T partner is the
// contiguous key run E g .. E g + E - 1 of one dim.
// ---------------------------------------------------------------------------
template <typename T>
struct KvLayout {
  static constexpr int E = Mma<T>::E, KB = Mma<T>::KSTEP, NBLK = KB / 16;
  static __host__ __device__ __forceinline__ int key_of(int blk, int r) { return E * (r / 4) + 4 * blk + r % 4; }
  // element offset of K[key][c] within one (request, head)'s cache of dh columns
  static __host__ __device__ __forceinline__ size_t k_off(int key, int c, int dh) {
    const int j = key / KB, kk = key % KB;
    const int r = 4 * (kk / E) + kk % 4, blk = (kk % E) / 4;
    const int nf = dh / KB, kf = c / KB, g = (c % KB) / E;
    return ((static_cast<size_t>(j) * NBLK * nf + blk * nf + kf) * 64 + g * 16 + r) * E + c % E;
  }
  // element offset of V[key][d]
  static __host__ __device__ __forceinline__ size_t v_off(int key, int d, int dh) {
    const int j = key / KB, kk = key % KB;
    return ((static_cast<size_t>(j) * (dh / 16) + d / 16) * 64 + (kk / E) * 16 + d % 16) * E + kk % E;
  }
  // elements of one key block of the K (or V) cache: KB * dh
  static __host__ __device__ __forceinline__ size_t block_elems(int dh) { return static_cast<size_t>(KB) * dh; }
};

// Pack 8 fp32 values into a bf16 fragment, or 4 fp32 values into an fp32 one.
__device__ __forceinline__ uint4 pack_frag_bf16(const float* v) {
  uint4 r;
  r.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
  r.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
  r.z = static_cast<uint32_t>(f2bf(v[4])) | (static_cast<uint32_t>(f2bf(v[5])) << 16);
  r.w = static_cast<uint32_t>(f2bf(v[6])) | (static_cast<uint32_t>(f2bf(v[7])) << 16);
  return r;
}

__device__ __forceinline__ uint4 pack_frag_f32(const float* v) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}

template <typename T> __device__ __forceinline__ uint4 pack_frag(const float* v);
template <> __device__ __forceinline__ uint4 pack_frag<bf16_t>(const float* v) { return pack_frag_bf16(v); }
template <> __device__ __forceinline__ uint4 pack_frag<float>(const float* v) { return pack_frag_f32(v); }

// Unpack a fragment into E fp32 values.
template <typename T> __device__ __forceinline__ void unpack_frag(uint4 f, float* v);
template <> __device__ __forceinline__ void unpack_frag<bf16_t>(uint4 f, float* v) {
  const uint32_t w[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void unpack_frag<float>(uint4 f, float* v) {
  v[0] = __uint_as_float(f.x); v[1] = __uint_as_float(f.y);
  v[2] = __uint_as_float(f.z); v[3] = __uint_as_float(f.w);
}

// Hardware base-2 exponential (one v_exp_f32).  Results below 2^-126 may
// flush to zero; in a softmax that only drops terms more than 2^126 times
// smaller than the largest one.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax slack (log2 units): the running reference max of a query
// only moves when a new score exceeds it by more than this, so the rescale
// of the output accumulators is skipped for almost every key block.  Terms
// then reach at most 2^kSoftmaxSlack; the final ratio is unchanged.
constexpr float kSoftmaxSlack = 8.0f;

// ---------------------------------------------------------------------------
// Reductions within a wave (64 lanes)
// ---------------------------------------------------------------------------


// Combine lane l with lane l ^ 32 (resp. l ^ 16) through gfx950's lane
// swaps (one VALU op each instead of a round trip through the LDS crossbar).
// Both partners get the same value: the lower lane's operand comes first.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The value of lane l ^ 16 (resp. l ^ 32).
__device__ __forceinline__ float xor16_swap(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// The value of lane l ^ 1 (resp. l ^ 2) (DPP quad permutes).
__device__ __forceinline__ float xor1_swap(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float xor2_swap(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
}

// Rotate within each 16-lane row by N lanes (DPP row_ror).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// Sum over the 16 lanes sharing l / 16 (one "row" of a 16x16 fragment):
// rotate-and-add by 8, 4, 2, 1 within the row, every lane ends with the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

// Sum over the wave (64 lanes), every lane ends with the sum.
__device__ __forceinline__ float wave_sum(float v) { return xor32_sum(xor16_sum(row16_sum(v))); }

// ---------------------------------------------------------------------------
// Cross-workgroup exchange (split-K / split-KV fix-up).
//
// Partials are written and read with relaxed device-scope atomic accesses,
// which are coherent across the XCDs' separate L2s on their own (they carry
// the device-scope cache policy).  An agent-scope release/acquire fence
// would instead write back / invalidate the whole L2 of the XCD, once per
// wave, which costs tens of microseconds per launch.  Ordering comes from
// waiting for this thread's outstanding memory operations before the
// workgroup arrives on the group counter; the last workgroup to arrive
// reads the partials only after its counter update returned.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev4(f32x4* p, f32x4 v) {
  float* q = reinterpret_cast<float*>(p);
  st_dev(q, v[0]); st_dev(q + 1, v[1]); st_dev(q + 2, v[2]); st_dev(q + 3, v[3]);
}
__device__ __forceinline__ f32x4 ld_dev4(const f32x4* p) {
  const float* q = reinterpret_cast<const float*>(p);
  return f32x4{ld_dev(q), ld_dev(q + 1), ld_dev(q + 2), ld_dev(q + 3)};
}

// Every workgroup of a group publishes its partial (st_dev), then arrives
// on the group's counter; the last to arrive reduces all partials in a fixed
// order (so the result does not depend on arrival order) and resets the
// counter to zero for the next launch.  Returns true in every thread of the
// last workgroup.
__device__ __forceinline__ bool arrive_last(int* counter, int expected, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = (old == expected - 1);
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// ---------------------------------------------------------------------------
// Device-coherent 16/8/4-byte buffer accesses (device-scope cache policy):
// what one workgroup stores this way, another workgroup on any XCD reads
// this way, once the store has been acknowledged.  Used for every
// activation exchanged between workgroups inside one launch.  Offsets are
// bytes from the resource base (< 2 GiB).
// ---------------------------------------------------------------------------

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kCohPolicy = 16;  // device scope

struct Coh {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ explicit Coh(const void* base)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000)) {}
  __device__ __forceinline__ uint4 ld16(uint32_t off) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCohPolicy));
  }
  __device__ __forceinline__ uint2 ld8(uint32_t off) const {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCohPolicy));
  }
  __device__ __forceinline__ uint32_t ld4(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCohPolicy);
  }
  __device__ __forceinline__ void st16(uint32_t off, uint4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCohPolicy);
  }
  __device__ __forceinline__ void st8(uint32_t off, uint2 v) const {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kCohPolicy);
  }
  __device__ __forceinline__ void st4(uint32_t off, uint32_t v) const {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kCohPolicy);
  }
  __device__ __forceinline__ void st2(uint32_t off, uint16_t v) const {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kCohPolicy);
  }
  __device__ __forceinline__ float ldf(uint32_t off) const { return __uint_as_float(ld4(off)); }
  __device__ __forceinline__ void stf(uint32_t off, float v) const { st4(off, __float_as_uint(v)); }
};

__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(k0 * (x + 0.044715f * x * x * x)));
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

}  // namespace ae
