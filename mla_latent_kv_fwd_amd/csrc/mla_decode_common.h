// mla_decode_common.h -- device helpers shared by the decode kernels of
// libmla_decode (bf16 and FP8 caches).  Internal to the library; included by one
// kernel source each, inside namespace mla { namespace { ... } }.
#pragma once

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
// Read-only for the whole kernel: reads through this address space become scalar
// loads, counted by lgkmcnt rather than vmcnt, so they never wait on the
// direct-to-LDS loads in flight.
#define CONST_AS __attribute__((address_space(4)))

// Load a plain struct of 32-bit fields through the constant address space.
template <typename T>
__device__ __forceinline__ T load_const(const void* p) {
  static_assert(sizeof(T) % 4 == 0, "32-bit fields only");
  T r;
  const int CONST_AS* s = (const int CONST_AS*)p;
  int* d = reinterpret_cast<int*>(&r);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); i++) d[i] = s[i];
  return r;
}

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kRowsPerBlock / kWaves;  // 16
constexpr int kDimTiles = kHeadDimV / 16;          // 32 16-wide output tiles
constexpr float kLazyRescale = 8.0f;               // log2 of the largest p kept unrescaled
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kRowsPerWave == 16, "one 16x16x32 MFMA column block per wave");

// s_waitcnt immediate for "vector memory counter <= n", other counters untouched.
#define VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// One direct-to-LDS 16-byte load per lane from base + voff (base: wave-uniform,
// in SGPRs): lane i writes LDS[m0 + 16 i].  The cache is read once per step, so
// its loads carry the non-temporal hint (measured: the attention kernel 1.5-3%
// faster, and the split partials it writes stay cached for the combine).  The hazard recognizer does not see
// inside inline asm, so the asm supplies the wait states itself: an LDS-DMA load
// reading M0 right after M0 is written needs 1, and a vector memory instruction
// reading an SGPR that a VALU instruction just wrote needs 5.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  // readfirstlane returns int: go through uint32_t so the low half is zero-extended.
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sbase = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// The lane index, hidden from the optimiser.  Per-lane address terms derived
// from it where they are used are recomputed there (a few VALU operations)
// instead of being hoisted and kept live across the segment loop, where they
// would push the wave past 256 registers.
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// Max / sum over the four 16-lane groups that share a row.
__device__ __forceinline__ float row_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A split piece of a row block: per row the normalised output O = o * inv in fp16
// as O / s, with s a power of two set from the row's largest |O| so that
// |O / s| < 2^15, plus s and the LSE.  Lane (q, n) of wave w holds dims
// 16 d + 4 q + i of row 16 w + n; the row's maximum is taken over its four 16-lane
// groups.  The rows are staged in LDS (1,040-byte rows, conflict-free for these
// writes) and leave as whole 1 KiB rows, 16 bytes per lane (measured: the step 1.8%
// faster than 8-byte stores straight from the accumulator layout).  `stage` is
// LDS that every wave is done with once all have arrived (the ring after the last
// chunk); pbase is the partial index of the row block's first row.  Called by
// every thread of the workgroup.
__device__ __forceinline__ void store_partial(const DecodeArgs& a, size_t pbase, char LDS_AS* stage,
                                              const f32x4_t (&o)[kDimTiles], float inv, float lse_v) {
  const int ol = opaque_lane();
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int n = ol & 15, oq = ol >> 4;
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < kDimTiles; d++)
#pragma unroll
    for (int r = 0; r < 4; r++) amax = fmaxf(amax, fabsf(o[d][r]));
  amax = row_max(amax) * inv;
  // k = 14 - floor(log2 amax), kept where both 2^k and 2^-k are normal floats.
  const int e = (int)((__float_as_uint(amax) >> 23) & 255) - 127;
  int k = 14 - e;
  k = k < -126 ? -126 : (k > 126 ? 126 : k);
  const float s_inv = __uint_as_float((uint32_t)(127 + k) << 23);
  const float s = __uint_as_float((uint32_t)(127 - k) << 23);
  const float f = inv * s_inv;
  constexpr int kPitch = kHeadDimV * 2 + 16;
  static_assert(kRowsPerBlock * kPitch <= 130 * 1024, "the staged row block fits in the ring");
  __syncthreads();   // every wave is done with the ring
  char LDS_AS* rowp = stage + (wv * kRowsPerWave + n) * kPitch + 8 * oq;
#pragma unroll
  for (int d = 0; d < kDimTiles; d++) {
    f16x4_t w;
#pragma unroll
    for (int r = 0; r < 4; r++) w[r] = (_Float16)(o[d][r] * f);
    *reinterpret_cast<f16x4_t LDS_AS*>(rowp + 32 * d) = w;
  }
  if (oq == 0) {
    const size_t pidx = pbase + wv * kRowsPerWave + n;
    reinterpret_cast<float*>(a.ws + a.lay.part_lse)[pidx] = lse_v;
    reinterpret_cast<float*>(a.ws + a.lay.part_scale)[pidx] = s;
  }
  __syncthreads();
  typedef int i32x4_st __attribute__((ext_vector_type(4)));
  char* pout = a.ws + a.lay.part_out + pbase * (kHeadDimV * 2);
  // kRowsPerBlock rows x 64 granules over the workgroup: thread x moves granule
  // x & 63 of rows x / 64 + (kThreads / 64) i, i = 0..15, read four at a time so
  // the LDS latency is paid four times rather than sixteen.
  constexpr int kRowStep = kThreads / 64;
  static_assert(kRowsPerBlock * (kHeadDimV * 2 / 16) == 16 * kThreads, "16 granules per thread");
  const int x0 = (int)threadIdx.x;
  const char LDS_AS* src = stage + (x0 >> 6) * kPitch + (x0 & 63) * 16;
  char* dst = pout + (size_t)(x0 >> 6) * (kHeadDimV * 2) + (x0 & 63) * 16;
#pragma unroll
  for (int h = 0; h < 4; h++) {
    i32x4_st v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = *reinterpret_cast<const i32x4_st LDS_AS*>(src + (4 * h + j) * kRowStep * kPitch);
#pragma unroll
    for (int j = 0; j < 4; j++) *reinterpret_cast<i32x4_st*>(dst + (4 * h + j) * kRowStep * (kHeadDimV * 2)) = v[j];
  }
}

// The same piece written straight from the accumulator layout (8-byte stores per
// lane), for a kernel with no registers to spare for the staging: pidx is the
// partial index of this lane's row.
__device__ __forceinline__ void store_partial_direct(const DecodeArgs& a, size_t pidx, int oq,
                                                     const f32x4_t (&o)[kDimTiles], float inv, float lse_v) {
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < kDimTiles; d++)
#pragma unroll
    for (int r = 0; r < 4; r++) amax = fmaxf(amax, fabsf(o[d][r]));
  amax = row_max(amax) * inv;
  const int e = (int)((__float_as_uint(amax) >> 23) & 255) - 127;
  int k = 14 - e;
  k = k < -126 ? -126 : (k > 126 ? 126 : k);
  const float s_inv = __uint_as_float((uint32_t)(127 + k) << 23);
  const float s = __uint_as_float((uint32_t)(127 - k) << 23);
  const float f = inv * s_inv;
  _Float16* prow = reinterpret_cast<_Float16*>(a.ws + a.lay.part_out) + pidx * kHeadDimV + 4 * oq;
#pragma unroll
  for (int d = 0; d < kDimTiles; d++) {
    f16x4_t w;
#pragma unroll
    for (int r = 0; r < 4; r++) w[r] = (_Float16)(o[d][r] * f);
    *reinterpret_cast<f16x4_t*>(prow + 16 * d) = w;
  }
  if (oq == 0) {
    reinterpret_cast<float*>(a.ws + a.lay.part_lse)[pidx] = lse_v;
    reinterpret_cast<float*>(a.ws + a.lay.part_scale)[pidx] = s;
  }
}

__device__ __forceinline__ bf16x8_t lds_read_b128(const char LDS_AS* p) {
  return *reinterpret_cast<const bf16x8_t LDS_AS*>(p);
}
__device__ __forceinline__ i16x4_t lds_read_tr16(const char LDS_AS* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4_t LDS_AS*>(const_cast<char LDS_AS*>(p)));
}

// The plan in the workspace does not belong to this call: every workgroup writes
// the defined empty result (out = 0, lse = -inf) for its share of the rows --
// requests stretch, stretch + nwg, ... and row block rb -- and nothing else is
// read.  8-byte stores: out is only required to be 8-byte aligned.
__device__ __forceinline__ void write_empty_rows(const DecodeArgs& a, int stretch, int rb) {
  Header* hdr = reinterpret_cast<Header*>(a.ws + a.lay.header);
  if (threadIdx.x == 0 && stretch == 0 && rb == 0) atomicOr(&hdr->flags, (uint32_t)MLA_FLAG_BAD_PLAN);
  const int r0 = rb * kRowsPerBlock;
  const int nr = a.rows - r0 < kRowsPerBlock ? a.rows - r0 : kRowsPerBlock;
  constexpr int kPieces = kHeadDimV / 4;   // 8-byte pieces per row
  for (int b = stretch; b < a.batch; b += a.nwg) {
    uint2* orow = reinterpret_cast<uint2*>(a.out + ((size_t)b * a.rows + r0) * kHeadDimV);
    for (int g = threadIdx.x; g < nr * kPieces; g += blockDim.x) orow[g] = make_uint2(0u, 0u);
    for (int r = threadIdx.x; r < nr; r += blockDim.x) a.lse[(size_t)b * a.rows + r0 + r] = -INFINITY;
  }
}
