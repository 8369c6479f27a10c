// mxfp4_resq.hip -- MXFP4 quantization with a Rollout-ResQ residual (K3)
// for gfx950.
//
// Method: "HiFloat4 Format for End-To-End Reinforcement Learning
// Post-Training of Large Language Models" (agifrontier.github.io), section
// on Rollout-ResQ and hardware-aware sparsity.  The rollout projection is
// rebuilt as Q(X)Q(W)^T + S(Q(dX))Q(W)^T with dX = X - Q(X); MXFP4 keeps
// one E8M0 scale per 32 E2M1 values; S_{2:4} keeps 2 of every 4
// consecutive values of the quantized residual.  This kernel produces
// Q(X), Q(dX)'s scale and its 2:4-compressed codes in one pass; the
// residual itself never leaves registers.
//
// Mapping: one lane per 8 elements, a quad of lanes per 32-element block.
#include "fp4q_device.h"
#include "fp4q_launch.h"

namespace fp4q {

namespace {

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Build-time knobs: FP4Q_MX_NT_STORES = 1 writes the outputs with
// non-temporal stores; FP4Q_MX_LDS_STAGE = 1 gathers a wavefront's outputs
// in LDS and writes them as 16-byte pieces.
#ifndef FP4Q_MX_LDS_STAGE
#define FP4Q_MX_LDS_STAGE 1
#endif
#ifndef FP4Q_MX_NT_LOADS
#define FP4Q_MX_NT_LOADS 1
#endif
#ifndef FP4Q_MX_NT_STORES
#define FP4Q_MX_NT_STORES 1
#endif
#ifndef FP4Q_MX_NT_SMALL
#define FP4Q_MX_NT_SMALL 0
#endif
// Build-time knobs: the cache-policy bits (see put) of the 16- and 4-byte
// outputs, and of the narrow ones (2 bytes or less per lane).
#ifndef FP4Q_MX_POLICY
#define FP4Q_MX_POLICY (FP4Q_MX_NT_STORES ? 2 : -1)
#endif
// Build-time knob: the cache-policy bits of the staged 16-byte pieces of
// the metadata and both scale outputs (256 and 64 bytes a wave).  sc1
// measured fastest on resq_act (29.2 us, dense 30.45) against nt (30.0,
// 30.7), none (29.3, 30.8) and nt with sc1 (30.0, 31.0); sc1 on the code
// and residual-code pieces as well was slower (30.6, 31.0).
#ifndef FP4Q_MX_STAGED_SMALL_POLICY
#define FP4Q_MX_STAGED_SMALL_POLICY 16
#endif
#ifndef FP4Q_MX_SMALL_POLICY
#define FP4Q_MX_SMALL_POLICY (FP4Q_MX_NT_STORES && FP4Q_MX_NT_SMALL ? 2 : -1)
#endif
template <typename T>
__device__ __forceinline__ void store_out(T* base, uint32_t idx, T v) {
  put<FP4Q_MX_POLICY>(base, idx, v);
}
template <typename T>
__device__ __forceinline__ void store_small(T* base, uint32_t idx, T v) {
  put<FP4Q_MX_SMALL_POLICY>(base, idx, v);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Max over the four lanes of a quad (the four lanes of one 32-element
// block): quad_perm [1,0,3,2], then [2,3,0,1].
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, dpp_mov<0xB1>(v));
  v = max(v, dpp_mov<0x4E>(v));
  return v;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// S_{2:4} choice for every group of four magnitude codes m0..m3 (3 bits
// each, index = m0 | m1 << 3 | m2 << 6 | m3 << 9): the two largest
// magnitudes, ties to the lower index; kept indices i0 < i1.  Entry bits
// 0-3: 4 i0, bits 4-7: 4 i1 (nibble offsets), bit 8: 0, bits 9-12:
// i0 | i1 << 2.
struct alignas(16) SelTable {
  uint16_t e[4096];
};
constexpr SelTable make_sel_table() {
  SelTable t{};
  for (int idx = 0; idx < 4096; ++idx) {
    int key[4] = {};
    for (int i = 0; i < 4; ++i) key[i] = ((idx >> (3 * i)) & 7) * 4 + (3 - i);
    int first = 0;
    for (int i = 1; i < 4; ++i)
      if (key[i] > key[first]) first = i;
    int second = first == 0 ? 1 : 0;
    for (int i = 0; i < 4; ++i)
      if (i != first && key[i] > key[second]) second = i;
    const int i0 = first < second ? first : second, i1 = first < second ? second : first;
    t.e[idx] = (uint16_t)((4 * i0) | ((4 * i1) << 4) | ((i0 | (i1 << 2)) << 9));
  }
  return t;
}
__device__ constexpr SelTable kSelTable = make_sel_table();

// S_{2:4} of one code word holding two groups of four nibbles (group 0 in
// the low 16 bits), through the table in LDS.  Returns the kept codes, two
// per group (lower index in the low nibble), and sets meta to i0 | i1 << 2
// per group (group 0 in the low nibble).
__device__ __forceinline__ uint32_t select_2of4(uint32_t rw, const uint16_t* tab,
                                                uint32_t& meta) {
  // gather the 3-bit magnitudes of each group into 12 bits, both groups at
  // once (group 0 in bits 0-11, group 1 in bits 16-27)
  const uint32_t t = (rw & 0x07070707u) | ((rw >> 1) & 0x38383838u);
  const uint32_t idx = (t & 0x003F003Fu) | ((t >> 2) & 0x0FC00FC0u);
  const uint32_t e0 = tab[idx & 0xFFFu], e1 = tab[idx >> 16];
  const uint32_t hi = rw >> 16;
  // the field offset uses the low 5 bits of its operand: e holds 4 i0 in
  // bits 0-3 with bit 4 (bit 0 of 4 i1) zero, and e >> 4 holds 4 i1 with
  // bit 4 (entry bit 8) zero
  const uint32_t n00 = __builtin_amdgcn_ubfe(rw, e0, 4);
  const uint32_t n01 = __builtin_amdgcn_ubfe(rw, e0 >> 4, 4);
  const uint32_t n10 = __builtin_amdgcn_ubfe(hi, e1, 4);
  const uint32_t n11 = __builtin_amdgcn_ubfe(hi, e1 >> 4, 4);
  meta = (e0 >> 9) | ((e1 >> 5) & 0xF0u);
  return n00 | (n01 << 4) | (n10 << 8) | (n11 << 12);
}

// Units of 8 elements (16 input bytes): a wavefront owns 64 * NU
// consecutive units and lane l takes units l, l + 64, ... of them, so every
// load instruction reads 1 KiB contiguously.  The four lanes of a quad hold
// one 32-element block per unit slot and share its scale through DPP.
#ifndef FP4Q_MX_UNITS
#define FP4Q_MX_UNITS 4
#endif
constexpr int kUnitsPerLane = FP4Q_MX_UNITS;
// Build-time knob: wavefronts per workgroup of the quantize kernels (4, 8 or
// 16); each workgroup copies the 8 KiB 2:4 table into LDS once.  Fewer
// table copies did not pay: resq_act 8192 x 7168 took 31.0 us with 8 and
// 33.9 us with 16 against 29.9 us with 4.
#ifndef FP4Q_MX_WG_WAVES
#define FP4Q_MX_WG_WAVES 4
#endif
constexpr int kMxWaves = FP4Q_MX_WG_WAVES;
static_assert(kMxWaves == 4 || kMxWaves == 8 || kMxWaves == 16, "4, 8 or 16 wavefronts");

// Build-time knob: FP4Q_STANDIN = 1 builds a memory-pattern stand-in for
// measurement only (libfp4q_standin.so, never the quantizer): the same
// loads, 2:4 table copy, staging and stores, with each unit's quantization
// and 2:4 selection replaced by XORs of its input words.
#ifndef FP4Q_STANDIN
#define FP4Q_STANDIN 0
#endif

// Build-time knob: FP4Q_MX_FLOAT_MAX = 1 takes each unit's max |x| from its
// widened FP32 values (three-input maxima of magnitudes; 4 fewer VALU
// instructions per unit, resq_act 29.96 -> 29.89 us, dense 30.73 -> 30.61
// us); 0: a packed 16-bit integer maximum of the sign-cleared BF16 words.
#ifndef FP4Q_MX_FLOAT_MAX
#define FP4Q_MX_FLOAT_MAX 1
#endif

__device__ __forceinline__ void resq_unit(const uint4 a, uint32_t& cw, uint32_t& rw, int& k,
                                          int& kr) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  float v[8];
  static_for<0, 4>([&](auto P) {
    constexpr int p = decltype(P)::value;
    v[2 * p] = bf16_lo(w[p]);
    v[2 * p + 1] = bf16_hi(w[p]);
  });
  uint32_t mbits;
  if (FP4Q_MX_FLOAT_MAX) {
    // primary scale: max |x| by three-input IEEE maxima of the widened
    // values, which return an operand unchanged: the bits are the
    // sign-cleared BF16 pattern shifted up (NaN is outside the domain)
    auto mx3 = [](float p, float q, float r) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(p, q), r);
    };
    float m = mx3(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]), __builtin_fabsf(v[2]));
    m = mx3(m, __builtin_fabsf(v[3]), __builtin_fabsf(v[4]));
    m = mx3(m, __builtin_fabsf(v[5]), __builtin_fabsf(v[6]));
    mbits = __float_as_uint(__builtin_elementwise_maximum(m, __builtin_fabsf(v[7])));
  } else {
    // primary scale: packed 16-bit max of the sign-cleared BF16 patterns
    const u16x2 mw = __builtin_elementwise_max(
        __builtin_elementwise_max(as_u16x2(w[0] & 0x7FFF7FFFu), as_u16x2(w[1] & 0x7FFF7FFFu)),
        __builtin_elementwise_max(as_u16x2(w[2] & 0x7FFF7FFFu), as_u16x2(w[3] & 0x7FFF7FFFu)));
    mbits = (uint32_t)max(mw.x, mw.y) << 16;
  }
  mbits = quad_max(mbits);
  k = mx_exponent(mbits);  // [-127, 125]
  const float up = __uint_as_float((uint32_t)(127 + k) << 23);  // 2^k as a scale operand

  // primary codes of x / 2^k, the division done inside the conversion
  cw = any_word();  // bytes 0-3 all written below
  static_for<0, 4>([&](auto P) {
    constexpr int p = decltype(P)::value;
    cw = cvt_e2m1x2_scaled<p>(cw, v[2 * p], v[2 * p + 1], up);
  });

  // residual x - (+-g 2^k), exact in FP32
  float rmax = 0.0f;
  static_for<0, 4>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const float2v g = e2m1x2_values_scaled<p>(cw, up);
    v[2 * p] = v[2 * p] - g.x;
    v[2 * p + 1] = v[2 * p + 1] - g.y;
    rmax = fmaxf(fmaxf(rmax, fabsf(v[2 * p])), fabsf(v[2 * p + 1]));
  });
  kr = mx_exponent(quad_max(__float_as_uint(rmax)));
  const float rup = __uint_as_float((uint32_t)(127 + kr) << 23);
  rw = any_word();
  static_for<0, 4>([&](auto P) {
    constexpr int p = decltype(P)::value;
    rw = cvt_e2m1x2_scaled<p>(rw, v[2 * p], v[2 * p + 1], rup);
  });
}

// DENSE = false: Rollout-ResQ with S_{2:4} (res_codes uint16 per unit,
// res_meta one byte per unit); DENSE = true: Rollout-ResQ-Dense (res_codes
// uint32 per unit, packed like the primary codes).
//
// Staged stores (stage != 0: every output 16-byte aligned; wave-uniform
// for a wavefront whose 64 * NU units all exist): the five outputs of the
// wavefront's units are contiguous ranges -- codes 4 bytes a unit, residual
// codes 2 (dense 4), metadata 1, each scale 1 per 4 units -- so they are
// gathered in the wavefront's LDS area, in that order, and leave as 16-byte
// pieces, each lane writing one piece of whichever output it falls in.
template <bool DENSE>
struct StageLayout {
  static constexpr int kCode = 16 * kUnitsPerLane;  // 16-byte pieces of each output
  static constexpr int kRes = (DENSE ? 16 : 8) * kUnitsPerLane;
  static constexpr int kMeta = DENSE ? 0 : 4 * kUnitsPerLane;
  static constexpr int kSc = kUnitsPerLane;
  static constexpr int kResAt = kCode, kMetaAt = kResAt + kRes, kScAt = kMetaAt + kMeta,
                       kRscAt = kScAt + kSc, kPieces = kRscAt + kSc;
};

template <bool DENSE>
__global__ __launch_bounds__(64 * kMxWaves) void mxfp4_resq_units(
    const uint4* __restrict__ x, int64_t u0, int64_t u_end, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, void* __restrict__ res_codes,
    uint8_t* __restrict__ res_meta, uint8_t* __restrict__ res_scales, int stage) {
  typedef StageLayout<DENSE> SL;
  __shared__ uint4 stage_lds[FP4Q_MX_LDS_STAGE ? kMxWaves * SL::kPieces : 1];
  __shared__ uint4 tab_lds[DENSE ? 1 : 512];
  const uint16_t* tab = reinterpret_cast<const uint16_t*>(tab_lds);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // first unit of this wave (uniform); u0 and u_end are multiples of 4, so
  // quads are whole
  const int64_t ub = u0 + ((int64_t)blockIdx.x * kMxWaves + wave) * 64 * kUnitsPerLane;
  const int64_t left = u_end - ub;  // units of this wave that exist (may be <= 0)
  // a wave past the end loads nothing but still writes its share of the
  // table and meets the barrier below before it leaves
  const int nv = left <= 0 ? 0 : left < 64 * kUnitsPerLane ? (int)left : 64 * kUnitsPerLane;
  const uint4* xw = x + ub;  // wave-uniform bases, 32-bit lane offsets
  uint32_t* cw_out = codes + ub;
  uint8_t* sc_out = scales + (ub >> 2);
  uint8_t* rs_out = res_scales + (ub >> 2);
  const bool staged = FP4Q_MX_LDS_STAGE && stage != 0 && nv == 64 * kUnitsPerLane;
  uint8_t* sb = reinterpret_cast<uint8_t*>(stage_lds + (FP4Q_MX_LDS_STAGE ? wave * SL::kPieces : 0));
  uint4 a[kUnitsPerLane];
#pragma unroll
  for (int n = 0; n < kUnitsPerLane; ++n)
    if (64 * n < nv) {
      const uint4* src = &xw[min(lane + 64 * n, nv - 1)];  // in bounds for every lane
      if (FP4Q_MX_NT_LOADS) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)src);
        a[n] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        a[n] = *src;
      }
    }
  // the 2:4 table (8 KiB) into LDS, its loads issued after the wave's own so
  // that the two latencies overlap (loading it first and waiting for it
  // before the input loads cost a second memory round trip per workgroup)
  if (!DENSE) {
    const uint4* tab_src = reinterpret_cast<const uint4*>(kSelTable.e);
    constexpr int kPer = 512 / (64 * kMxWaves);  // 16-byte table pieces per thread
    uint4 t[kPer > 0 ? kPer : 1];
#pragma unroll
    for (int k = 0; k < kPer; ++k) t[k] = tab_src[threadIdx.x + 64 * kMxWaves * k];
    if (kPer == 0 && threadIdx.x < 512) t[0] = tab_src[threadIdx.x];
#pragma unroll
    for (int k = 0; k < kPer; ++k) tab_lds[threadIdx.x + 64 * kMxWaves * k] = t[k];
    if (kPer == 0 && threadIdx.x < 512) tab_lds[threadIdx.x] = t[0];
    __syncthreads();
  }
  if (nv == 0) return;
#pragma unroll
  for (int n = 0; n < kUnitsPerLane; ++n) {
    const int j = lane + 64 * n;
    if (64 * n < nv) {  // wave-uniform
      uint32_t cw, rw;
      int k, kr;
      if (FP4Q_STANDIN) {
        cw = a[n].x ^ a[n].z;
        rw = a[n].y ^ a[n].w;
        k = (int)(a[n].x >> 25) - 127;
        kr = (int)(a[n].y >> 25) - 127;
      } else {
        resq_unit(a[n], cw, rw, k, kr);
      }
      if (staged) {
        reinterpret_cast<uint32_t*>(sb)[j] = cw;
        if (DENSE) {
          reinterpret_cast<uint32_t*>(sb + 16 * SL::kResAt)[j] = rw;
        } else {
          uint32_t meta = rw >> 24;
          const uint32_t rc = FP4Q_STANDIN ? rw : select_2of4(rw, tab, meta);
          reinterpret_cast<uint16_t*>(sb + 16 * SL::kResAt)[j] = (uint16_t)rc;
          sb[16 * SL::kMetaAt + j] = (uint8_t)meta;
        }
        if ((lane & 3) == 0) {
          sb[16 * SL::kScAt + (j >> 2)] = (uint8_t)(k + 127);
          sb[16 * SL::kRscAt + (j >> 2)] = (uint8_t)(kr + 127);
        }
        continue;
      }
      if (DENSE) {
        if (j < nv) store_out(reinterpret_cast<uint32_t*>(res_codes) + ub, j, rw);
      } else {
        uint32_t meta = rw >> 24;
        const uint32_t rc = FP4Q_STANDIN ? rw : select_2of4(rw, tab, meta);
        if (j < nv) {
          store_small(reinterpret_cast<uint16_t*>(res_codes) + ub, j, (uint16_t)rc);
          store_small(res_meta + ub, j, (uint8_t)meta);
        }
      }
      if (j < nv) {
        store_out(cw_out, j, cw);
        if ((lane & 3) == 0) {
          store_small(sc_out, j >> 2, (uint8_t)(k + 127));
          store_small(rs_out, j >> 2, (uint8_t)(kr + 127));
        }
      }
    }
  }
  if (staged) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint4* st = stage_lds + wave * SL::kPieces;
    // each output's first piece (wave-uniform)
    uint4* const o_code = reinterpret_cast<uint4*>(cw_out);
    uint4* const o_res =
        reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(res_codes) + ub * (DENSE ? 4 : 2));
    uint4* const o_meta = reinterpret_cast<uint4*>(DENSE ? nullptr : res_meta + ub);
    uint4* const o_sc = reinterpret_cast<uint4*>(sc_out);
    uint4* const o_rs = reinterpret_cast<uint4*>(rs_out);
#pragma unroll
    for (int p0 = 0; p0 < SL::kPieces; p0 += 64) {
      const int p = p0 + lane;
      if (p < SL::kResAt)
        store_out(o_code, p, st[p]);
      else if (p < SL::kMetaAt)
        store_out(o_res, p - SL::kResAt, st[p]);
      else if (p < SL::kScAt)
        put<FP4Q_MX_STAGED_SMALL_POLICY>(o_meta, p - SL::kMetaAt, st[p]);
      else if (p < SL::kRscAt)
        put<FP4Q_MX_STAGED_SMALL_POLICY>(o_sc, p - SL::kScAt, st[p]);
      else if (p < SL::kPieces)
        put<FP4Q_MX_STAGED_SMALL_POLICY>(o_rs, p - SL::kRscAt, st[p]);
    }
  }
}

// The residual of one unit as a dense code word: the two kept codes of each
// group of four at the positions their metadata names, zeros elsewhere.
__device__ __forceinline__ uint32_t expand_2of4(uint32_t rc, uint32_t meta) {
  uint32_t w = 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t kb = (rc >> (8 * h)) & 0xFFu, m = (meta >> (4 * h)) & 15u;
    w |= ((kb & 15u) << (4 * (m & 3u) + 16 * h)) | ((kb >> 4) << (4 * (m >> 2) + 16 * h));
  }
  return w;
}

// X_hat = DQ(Q(X)) (+ the residual): one lane per 8-element unit; every
// dequantized value is +-g 2^k, exact through the scaled decode, and the
// two terms are added once in FP32.  A wavefront's 64 units are 2 KiB of
// output: with FP4Q_MX_REC_STAGE each lane puts its 32 bytes in the wave's
// LDS area and the wave writes them back as two 1 KiB contiguous store
// instructions (waves at a ragged end store lane by lane).
#ifndef FP4Q_MX_REC_STAGE
#define FP4Q_MX_REC_STAGE 1
#endif
#ifndef FP4Q_MX_REC_NT
#define FP4Q_MX_REC_NT 1
#endif
// Build-time knob: the cache-policy bits (see put) of the FP32 output: nt
// with sc1 measured 41.0 against 41.4 us for nt alone on the 8192 x 7168
// S2:4 reconstruction (sc1 gained nothing on the quantizer's outputs).
#ifndef FP4Q_MX_REC_POLICY
#define FP4Q_MX_REC_POLICY (FP4Q_MX_REC_NT ? 18 : -1)
#endif
__device__ __forceinline__ void store_rec(uint4* base, uint32_t idx, uint4 v) {
  put<FP4Q_MX_REC_POLICY>(base, idx, v);
}
template <int RES>
__global__ __launch_bounds__(256) void mxfp4_reconstruct_units(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const void* __restrict__ res_codes, const uint8_t* __restrict__ res_meta,
    const uint8_t* __restrict__ res_scales, int64_t u0, int64_t u_end,
    uint4* __restrict__ out) {
  __shared__ uint4 stage_lds[FP4Q_MX_REC_STAGE ? 512 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t uw = u0 + (int64_t)blockIdx.x * 256 + 64 * wave;  // the wave's first unit
  const int64_t u = uw + lane;
  const bool staged = FP4Q_MX_REC_STAGE && uw + 64 <= u_end;
  if (u >= u_end) return;
  const uint32_t cw = codes[u];
  const float up = __uint_as_float((uint32_t)scales[u >> 2] << 23);  // E8M0 as a scale operand
  uint32_t rw = 0u;
  float rup = 0.0f;
  if (RES == 2) rw = reinterpret_cast<const uint32_t*>(res_codes)[u];
  if (RES == 1) rw = expand_2of4(reinterpret_cast<const uint16_t*>(res_codes)[u], res_meta[u]);
  if (RES != 0) rup = __uint_as_float((uint32_t)res_scales[u >> 2] << 23);
  uint32_t o[8];
  static_for<0, 4>([&](auto P) {
    constexpr int p = decltype(P)::value;
    float2v v = e2m1x2_values_scaled<p>(cw, up);
    if (RES != 0) v = v + e2m1x2_values_scaled<p>(rw, rup);
    o[2 * p] = __float_as_uint(v.x);
    o[2 * p + 1] = __float_as_uint(v.y);
  });
  if (staged) {
    uint4* st = stage_lds + 128 * (threadIdx.x >> 6);
    st[2 * lane] = make_uint4(o[0], o[1], o[2], o[3]);
    st[2 * lane + 1] = make_uint4(o[4], o[5], o[6], o[7]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    store_rec(out + 2 * uw, lane, st[lane]);
    store_rec(out + 2 * uw, 64 + lane, st[64 + lane]);
  } else {
    store_rec(out + 2 * uw, 2 * lane, make_uint4(o[0], o[1], o[2], o[3]));
    store_rec(out + 2 * uw, 2 * lane + 1, make_uint4(o[4], o[5], o[6], o[7]));
  }
}

}  // namespace

template <bool DENSE>
hipError_t resq_launch(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                       uint8_t* scales, void* res_codes, uint8_t* res_meta, uint8_t* res_scales,
                       hipStream_t st) {
  const int64_t nunits = rows * (hidden / 8);  // a multiple of 4
  const int64_t max_units = FP4Q_MAX_LAUNCH_ITEMS / 256 * 256 * kUnitsPerLane;
  const auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const int stage = a16(codes) && a16(scales) && a16(res_codes) && a16(res_scales) &&
                    (DENSE || a16(res_meta));
  for (int64_t u0 = 0; u0 < nunits; u0 += max_units) {
    const int64_t n = nunits - u0 < max_units ? nunits - u0 : max_units;
    constexpr int64_t per_wg = 64 * kMxWaves * kUnitsPerLane;
    const dim3 grid((unsigned)((n + per_wg - 1) / per_wg)), block(64 * kMxWaves);
    hipLaunchKernelGGL(mxfp4_resq_units<DENSE>, grid, block, 0, st, (const uint4*)x, u0, u0 + n,
                       (uint32_t*)codes, scales, res_codes, res_meta, res_scales, stage);
  }
  return hipGetLastError();
}

hipError_t mxfp4_resq_launch(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                             uint8_t* scales, uint8_t* res_codes, uint8_t* res_meta,
                             uint8_t* res_scales, hipStream_t st) {
  return resq_launch<false>(x, rows, hidden, codes, scales, res_codes, res_meta, res_scales, st);
}

hipError_t mxfp4_resq_dense_launch(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                                   uint8_t* scales, uint8_t* res_codes, uint8_t* res_scales,
                                   hipStream_t st) {
  return resq_launch<true>(x, rows, hidden, codes, scales, res_codes, nullptr, res_scales, st);
}

hipError_t mxfp4_reconstruct_launch(const uint8_t* codes, const uint8_t* scales,
                                    const uint8_t* res_codes, const uint8_t* res_meta,
                                    const uint8_t* res_scales, int64_t rows, int64_t hidden,
                                    int residual, float* out, hipStream_t st) {
  const int64_t nunits = rows * (hidden / 8);
  const int64_t max_units = FP4Q_MAX_LAUNCH_ITEMS / 256 * 256;
  for (int64_t u0 = 0; u0 < nunits; u0 += max_units) {
    const int64_t n = nunits - u0 < max_units ? nunits - u0 : max_units;
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (residual == 2)
      hipLaunchKernelGGL(mxfp4_reconstruct_units<2>, grid, block, 0, st, (const uint32_t*)codes,
                         scales, res_codes, res_meta, res_scales, u0, u0 + n, (uint4*)out);
    else if (residual == 1)
      hipLaunchKernelGGL(mxfp4_reconstruct_units<1>, grid, block, 0, st, (const uint32_t*)codes,
                         scales, res_codes, res_meta, res_scales, u0, u0 + n, (uint4*)out);
    else
      hipLaunchKernelGGL(mxfp4_reconstruct_units<0>, grid, block, 0, st, (const uint32_t*)codes,
                         scales, res_codes, res_meta, res_scales, u0, u0 + n, (uint4*)out);
  }
  return hipGetLastError();
}

}  // namespace fp4q
