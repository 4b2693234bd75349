// Device helpers shared by the gfx950 kernels: bf16 vectors, MFMA wrappers,
// LDS transpose reads and the workspace layout.
//
// MFMA lane layouts (v_mfma_f32_32x32x16_bf16, wave64), with l = lane id,
// g = l / 32:
//   A (32 x 16, M x K): lane l holds A[l % 32][8g .. 8g+7]
//   B (16 x 32, K x N): lane l holds B[8g .. 8g+7][l % 32]
//   C (32 x 32):        lane l, register r holds C[8(r/4) + 4g + r%4][l % 32]
// Since A and B are both "8 contiguous K values for one fixed non-K index",
// a C tile can feed the next product as either operand with its *row* index
// as the contraction index, provided the other operand uses the same
// permutation of K: lane group g then holds rows {4g..4g+3, 8+4g..8+4g+3} of
// each 16-row slice (registers 8h..8h+7 of the accumulator for slice h).
//
// ds_read_b64_tr_b16 (gfx950) works on groups of 16 lanes: output lane i,
// element t receives element (i & 3) of the 64-bit word addressed by lane
// 4t + (i >> 2) of its group. If lane s of a group addresses row k0 + s/4,
// columns c0 + 4(s%4) .. +3 of a row-major bf16 matrix M, output lane i gets
// M[k0 .. k0+3][c0 + i]: a 4 x 16 block read transposed. Two such reads give
// the 8 K values an MFMA operand lane needs from a matrix stored K-major.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

static constexpr float kLog2e = 1.4426950408889634f;

// Buffer resources (raw, stride 0): fourth descriptor word selecting 32-bit
// data, and the cache-policy bits of the buffer access builtins (sc0: coherent
// in the XCD's L2; sc1: coherent across XCDs).
static constexpr int kBufferWord3 = 0x00020000;
static constexpr int kBufSc0 = 1;
static constexpr int kBufSc1 = 16;

// The fp32 dQ accumulator of the read-modify-write modes is kept in MFMA
// fragment order (the atomic modes keep it row-major): rows in 32-row
// blocks, each block as D/32 column blocks of 32 x 32; inside such a block the
// element (row 8h + 4g + e, column c) sits at float (h * 64 + 32g + c) * 4 + e,
// so one lane's four accumulator registers 4h .. 4h+3 are 16 contiguous bytes.

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  r[2] = (__bf16)c;
  r[3] = (__bf16)d;
  return r;
}

// Two fp32 -> two bf16 (RNE) with one v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x2 cvt2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, bf16x2); }

// 16-byte LDS load/store.
__device__ __forceinline__ bf16x8 lds_load16(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void lds_store16(__bf16* p, const bf16x8& v) { *reinterpret_cast<bf16x8*>(p) = v; }

// Transposed 4x16 read (see header): `p` is this lane's 64-bit source address.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    r[t] = a[t];
    r[4 + t] = b[t];
  }
  return r;
}

// Operand fragment of a row-major bf16 matrix M (pitch in elements), read
// K-major: lane holds M[k0 + rows(g)][c0 + l%32] for the 8 K rows its group
// needs. `perm` selects the accumulator-compatible K permutation
// ({4g..4g+3, 8+4g..8+4g+3}); otherwise K rows 8g..8g+7 in order.
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* M, int pitch, int k0, int c0, bool perm) {
  const int l = threadIdx.x & 63;
  const int s = l & 15;           // lane within its 16-lane group
  const int grp = l >> 4;         // 0..3
  const int g = grp >> 1;         // K half
  const int cbase = c0 + 16 * (grp & 1) + 4 * (s & 3);
  int ka, kb;
  if (perm) {
    ka = k0 + 4 * g + (s >> 2);
    kb = ka + 8;
  } else {
    ka = k0 + 8 * g + (s >> 2);
    kb = ka + 4;
  }
  bf16x4 lo = lds_read_tr(M + ka * pitch + cbase);
  bf16x4 hi = lds_read_tr(M + kb * pitch + cbase);
  return cat(lo, hi);
}

// Operand fragment of a row-major bf16 matrix read along its rows: lane holds
// M[r0 + l%32][k0 + 8g .. +7].
__device__ __forceinline__ bf16x8 frag_row(const __bf16* M, int pitch, int r0, int k0) {
  const int l = threadIdx.x & 63;
  return lds_load16(M + (r0 + (l & 31)) * pitch + k0 + 8 * (l >> 5));
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles. A tile of R rows x (NCH 16-byte chunks) is stored without
// padding; logical chunk c of row r sits at physical chunk c ^ swz_f<NCH>(r).
// The XOR pattern makes both access patterns used on these tiles hit distinct
// LDS banks (64 banks x 4 bytes): 16 consecutive rows read at one chunk
// (16-byte row fragments), and 4 consecutive rows x 4 consecutive chunks
// (transpose reads of two 16-lane groups).
// ---------------------------------------------------------------------------
template <int NCH>
__device__ __forceinline__ int swz_f(int r) {
  static_assert(NCH == 8 || NCH == 16, "rows of 128 or 256 bytes");
  if constexpr (NCH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// Asynchronous copy of n (a multiple of 64) fp32 values to LDS, by wave `wv`.
__device__ __forceinline__ void dma_f32(float* lds, const float* __restrict__ gsrc, int n, int wv) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (w != wv) return;
  for (int x = 0; x < n; x += 64)
    __builtin_amdgcn_global_load_lds((gbl_void*)(gsrc + x + lane), (lds_void*)(lds + x), 4, 0, 0);
}

__device__ __forceinline__ void wait_vm_all() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workspace header (32-bit words). The preprocess kernel zeroes words
// [0, kHdrZeroWords) at the start of every call; the sticky status and its
// tag survive calls.
//   kHdrTicket      dynamic item counter of the ticket dispatch
//   kHdrAbort       error bits of the current call: a wait that sees it set
//                   gives up at once, so a failing call drains quickly
//   kHdrSticky      error bits of every call since the status was last read
//                   (detattn_device_status reads and clears them)
//   kHdrTag         two words: kStickyTag once the sticky word was initialised
static constexpr int kHdrTicket = 0;
static constexpr int kHdrAbort = 16;
static constexpr int kHdrZeroWords = 48;
static constexpr int kHdrSticky = 48;
static constexpr int kHdrTag = 50;
static constexpr unsigned long long kStickyTag = 0x5354494b59444154ull;

// Workspace layout (all offsets in bytes from the workspace base).
struct WsLayout {
  static constexpr size_t kHeader = 256;         // the header words above
  static constexpr size_t kMaxXcdGrid = 1024;    // workgroups the XCD registration table holds
  static constexpr size_t kXcdTab = kMaxXcdGrid * 4;
  static constexpr size_t kFlagStride = 128;     // one L2 line per dQ tile flag
  static constexpr size_t kMinBlockQ = 64;
  size_t xcdtab_off, flags_off, flags_bytes, ndelta_off, row_bytes, nlse_off, dqacc_off, dqacc_bytes, total;
  __host__ __device__ WsLayout(long long BH, long long S, long long D) {
    xcdtab_off = kHeader;
    flags_off = kHeader + kXcdTab;
    long long nq_max = (S + (long long)kMinBlockQ - 1) / (long long)kMinBlockQ;
    flags_bytes = (size_t)(BH * nq_max) * kFlagStride;
    ndelta_off = align(flags_off + flags_bytes);  // -D per row
    row_bytes = (size_t)(BH * S) * 4;
    nlse_off = align(ndelta_off + row_bytes);     // -LSE / scale per row
    dqacc_off = align(nlse_off + row_bytes);
    dqacc_bytes = (size_t)(BH * S * D) * 4;
    total = align(dqacc_off + dqacc_bytes);
  }
  __host__ __device__ static size_t align(size_t x) { return (x + 255) & ~(size_t)255; }
};

enum DeviceError : uint32_t { kErrNone = 0, kErrTimeout = 1 };

}  // namespace detattn
