// Bidirectional FAVOR+ in one persistent kernel (bf16 inputs, d = 64, m = 256).
//
// FA-part equation of the "FAVOR+" method page: O = D^-1 (Q' ((K')^T V)),
// D = diag(Q' ((K')^T 1_L)), with the positive features
// phi(x) = exp(w . x - |x|^2 / 2) / sqrt(m) (Gaussian kernel: -|x|^2 on the
// key side; ReLU features: max(w . x, 0), no norm term).
//
// Two launches per call:
//
//   fprep   W' = W log2(e) in fp16 (the projection operand of both sides) and
//           the control block of the persistent kernel cleared (a fill
//           kernel: no memset node when the call is captured in a graph).
//   fused   one work-group of 8 waves per compute unit.  Heads are dealt to
//           the eight accelerator dies (XCDs, each with its own L2) in turn;
//           each die has a queue of key items and a queue of query items for
//           its heads.  A work-group claims key items (its die's first,
//           then the other dies') until every key queue is empty, then query
//           items the same way.  A key item (head, split) computes the
//           partial state [(K')^T V | (K')^T 1] of one split of the head's
//           tokens over all 256 features: its two groups of four waves take
//           alternate 32-token tiles, the four waves of a group one
//           64-feature block each, sharing the tile's K and V through LDS.
//           It writes the partial in fp32 with its per-feature references and
//           arrives at the head.  A query item (head, query block) stages W',
//           waits for the head's splits, sums their partials into the bf16
//           state and applies it to its tokens.  A work-group starts query
//           items only once every key item has been taken by a running
//           work-group, and key items wait for nothing: every wait ends.
//
// The key exponent needs no reference on the fast path.  With
// W' = W log2(e), the key feature's exponent is
//   e = k . w' - knorm |k|^2 log2(e) = log2(e) (|w|^2/2 - |k - w|^2/2)
// for knorm = 1/2 (|w|^2/4 - |k - w/2|^2 for knorm = 1), so
// e <= log2(e) |w|^2 / 2 whatever k is: the features cannot overflow, and
// the norm term enters the projection as the matrix instruction's C input.
// The query side likewise uses its own norm as the per-row shift (it cancels
// in D^-1).  Robustness: a key item whose sums are not finite, or whose ones
// column underflows (keys far from every projection row), is redone with
// per-feature references (set from each wave's first tile, raised lazily),
// and a query tile whose denominators leave [2^-100, 2^100] (or whose head
// carries references) is redone with a per-row reference from its exact row
// maximum.  Every shift is exact: per-feature key shifts are compensated on
// the query exponent, per-row query shifts cancel in D^-1.  The slow forms
// run the same code as the fast ones with a flag (the kernel makes no
// function calls: a kernel that calls keeps a stack in scratch memory).
//
// Exchange between work-groups: partial states, references and arrival
// counts are written with device-scope (sc1) stores, which write through to
// the device's coherence point, and read with device-scope loads; a
// work-group waits for its stores to complete (vmcnt 0) before it signals
// with a device-scope atomic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "favor.h"
#include "favor_internal.h"
#include "mfma_common.h"

namespace favor {
namespace {

using namespace mfma;

constexpr int FD = 64;            // head dimension
constexpr int FM = 256;           // features
constexpr int FTT = 32;           // tokens per tile
constexpr int FNT = 512;          // threads per work-group (8 waves)
constexpr int NW = FNT / 64;      // waves per work-group
constexpr int NTG = 2;            // token groups of a key item
constexpr int NFW = NW / NTG;     // waves per token group (one 64-feature block each)
constexpr int NSPLIT = 4;         // at most this many key items (splits) per head
constexpr int FNCH = FM / 64;     // 64-feature chunks of the query side
constexpr int WROW = FD + 8;      // fp16 per W' row (workspace and LDS)
constexpr int KZROW = FM + 8;     // bf16 per state row (LDS)
constexpr int KZROWS = FD + 16;   // state rows: 64 value columns, z, zero rows to 80
constexpr int PROWS = FD + 1;     // rows of a partial state (value columns, z)
constexpr int QTILE = 32;         // tokens per query tile (two 16-token columns)
constexpr int NXCD = 8;           // accelerator dies of the part

constexpr float kKeyBiasF = 40.0f;   // slow key loop: features start at <= 2^-40
constexpr unsigned kSpinLimit = 1u << 25;   // ~1 s of polling before giving up

// LDS of the key phase: per token group a six-slot ring of tiles, a slot
// holding K (bf16 as it lands, fp16 once converted), V ([32][64] rows of 128
// bytes, the 16-byte units of row r XOR-swizzled by r & 7) and the tile's 32
// norm terms; the merge slots of the second group's waves (20 accumulator
// quads and the references per lane) over the same bytes.
constexpr int KT_BYTES = FTT * FD * 2;
constexpr int SLOT_NB = 2 * KT_BYTES;
constexpr int SLOT_BYTES = 2 * KT_BYTES + FTT * 4;
constexpr int NSLOT = 6;
constexpr int RING_BYTES = NTG * NSLOT * SLOT_BYTES;
constexpr int MERGE_SLOT = 21 * 64 * 16;
constexpr int MERGE_BYTES = NFW * MERGE_SLOT;
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int KPHASE_BYTES = cmax(RING_BYTES, MERGE_BYTES);
// The query phase: W' [256][72] fp16, the state [80][264] bf16, the combined
// references c [256] fp32, the splits' scale factors [4][256] fp32.
constexpr int QW_BYTES = FM * WROW * 2;
constexpr int QK_BYTES = KZROWS * KZROW * 2;
constexpr int QC_BYTES = FM * 4;
constexpr int QS_BYTES = NSPLIT * FM * 4;
constexpr int QPHASE_BYTES = QW_BYTES + QK_BYTES + QC_BYTES + QS_BYTES;
constexpr int FUSED_LDS = cmax(KPHASE_BYTES, QPHASE_BYTES) + 64;
static_assert(FUSED_LDS <= 160 * 1024, "LDS of one work-group");

// Control block (u32, in the workspace): per die a key-queue and a
// query-queue head, a timeout flag, then per head the arrival count of its
// splits; each word on a 128-byte line of its own (atomics on one line from
// many work-groups serialize).
struct Ctrl {
  static constexpr int LINE = 32, TIMEOUT = 2 * NXCD * LINE, HEADS = 2 * NXCD + 4;
  __device__ static int kq(int x) { return x * LINE; }
  __device__ static int qq(int x) { return (NXCD + x) * LINE; }
  __device__ static int arrive(int bh) { return (HEADS + bh) * LINE; }
};
static_assert(Ctrl::HEADS == 20, "the control block's size is stated in favor_internal.h");

// Device-scope (sc1) accesses: cache policy bit 4 of the buffer and
// LDS-DMA instructions on this architecture.
constexpr int kSC1 = 16;

__device__ inline void store_sc1(unsigned* p, unsigned x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned load_sc1(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint4 load16_sc1(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline float load4_sc1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSC1));
}
__device__ inline void store4_sc1(__amdgpu_buffer_rsrc_t r, int off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, off, 0, kSC1);
}
// This wave's outstanding memory operations have completed.
__device__ inline void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// ---------------------------------------------------------------------------
// fprep: W16 [m][72] = fp16(W log2 e) (pad columns zero), control cleared.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fprep(const float* __restrict__ W,
                                             _Float16* __restrict__ W16,
                                             unsigned* __restrict__ ctrl, int nctrl) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < FM * WROW) {
    const int f = i / WROW, a = i - f * WROW;
    W16[i] = static_cast<_Float16>(a < FD ? W[f * FD + a] * kLog2e : 0.f);
  }
  for (int j = i; j < nctrl; j += gridDim.x * 256) ctrl[j] = 0u;
}

struct Args {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const _Float16* W16;
  const float* W32;  // the causal key kernel: W fp32, converted on load
  uint16_t* O;
  float* T;          // [BH][nsplit][65][256] partial states, fp32
  float* cs;         // [BH][nsplit][256] their per-feature references
  unsigned* ctrl;
  int L, BH, nsplit, seg, nqb, QB;
  float knorm;
};

// The work-group's LDS, shared by the key and query phases, and the last 64
// bytes as a broadcast area for values one thread decides.
__shared__ __align__(16) unsigned char g_smem[FUSED_LDS];
__device__ inline unsigned* bcast() { return reinterpret_cast<unsigned*>(g_smem + FUSED_LDS - 64); }
// LDS at byte offset `a` into the work-group's LDS (offsets formed once per
// lane, constants added at each use).  (An LDS pointer made from an integer
// would turn offset 0 into the null LDS pointer.)
template <class T>
__device__ inline __attribute__((address_space(3))) T* lds_at(uint32_t a) {
  return (__attribute__((address_space(3))) T*)((__attribute__((address_space(3))) unsigned char*)g_smem + a);
}
// The LDS address of g_smem (for instructions written out in assembly).
__device__ inline uint32_t lds_addr0() {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)g_smem));
}

// Sum over the four lanes {l, l^16, l^32, l^48} (one column of a 16x16 tile).
__device__ inline float colsum4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Instruction order for the scheduler in the region since the last
// scheduling barrier: P matrix instructions (a projection), then C matrix
// instructions each followed by up to V vector instructions (the features of
// the projected tile, which depend on the projection only), so that the
// vector units work while the matrix cores do.
template <int P, int C, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
#pragma unroll
  for (int k = 0; k < C; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

// Thread 0: the queue heads of every die (device-scope loads, issued while
// an item runs; a queue seen empty stays empty).
__device__ inline void take_snapshot(unsigned* q, unsigned (&c)[NXCD]) {
#pragma unroll
  for (int x = 0; x < NXCD; ++x) c[x] = load_sc1(q + Ctrl::LINE * x);
}

// Weight of a partial with reference c in a sum referred to cn >= c (a part
// that saw no token has c = -inf and weight 0).
__device__ inline float rescale(float c, float cn) {
  return c == -INFINITY ? 0.f : fast_exp2(c - cn);
}

// ---------------------------------------------------------------------------
// Key pass of one wave over its token group's tiles of the split [t0, t1)
// (group tg takes tiles tg, tg + 2, ...; the wave takes the 64 features
// 64 fw .. + 63, W' operands in registers).  Per step the work-group
// synchronises once.  Every wave DMAs a quarter of its group's tile five
// tiles ahead (waves fw = 0, 1 the K rows, 2, 3 the V rows) and converts a
// quarter of the K rows two tiles ahead in place to fp16, with those
// tokens' norm terms -knorm |k|^2 log2(e) (-inf past the split) beside the
// tile: each K element is converted once, not once per feature block.  Per
// tile: S = K W'^T - n on the matrix cores (the norm as the C input; the
// slow form subtracts the reference c_r there too), K~ = exp2(S) in bf16,
// and [V | 1]^T K~ accumulated in fp32, V read back as the contraction's
// operand with transposing LDS reads (4 consecutive tokens of one column per
// read).  Step i converts tile i + 2, projects tile i + 1 and contracts tile
// i.
// ---------------------------------------------------------------------------
//
// SEP: the two token groups take separate ranges instead (the caller passes
// each group its own [t0, t1), possibly empty), every tile of its range in
// order, both for ceil(nmax / 32) steps (a shorter range runs dead tiles);
// W' is converted from the fp32 W (a.W32) as it is loaded.
template <bool RELU, bool SLOW, bool SEP = false>
__device__ __forceinline__ void key_pass(const Args& a, int bh, int t0, int t1,
                                         f32x4 (&acc)[5][4], float (&cref)[4], int nmax = 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6), tg = wave / NFW, fw = wave % NFW;
  const int l16 = lane & 15, g = lane >> 4;
  unsigned char* const ring = g_smem + tg * NSLOT * SLOT_BYTES;
  const int n = t1 - t0;
  const int ntl = (n + FTT - 1) / FTT;      // tiles of the split
  // tiles per group (interleaved: group 1 may run one dead tile)
  const int nsteps = SEP ? (nmax + FTT - 1) / FTT : (ntl + NTG - 1) / NTG;
  const size_t base = (static_cast<size_t>(bh) * a.L + t0) * FD;
  const __amdgpu_buffer_rsrc_t rsrc_kv = buffer_rsrc((fw < 2 ? a.K : a.V) + base, n * FD * 2);
  const float nscale = -(a.knorm * kLog2e);
  // first token of the group's tile i, relative to t0
  auto tile_base = [&](int i) { return SEP ? i * FTT : (NTG * i + tg) * FTT; };

  f16x8 wb[4][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (SEP) {
        const float* wr = a.W32 + (64 * fw + 16 * nt + l16) * FD + 32 * ks + 8 * g;
        const float4 x = *reinterpret_cast<const float4*>(wr);
        const float4 y = *reinterpret_cast<const float4*>(wr + 4);
        f16x8 h;
        h[0] = static_cast<_Float16>(x.x * kLog2e); h[1] = static_cast<_Float16>(x.y * kLog2e);
        h[2] = static_cast<_Float16>(x.z * kLog2e); h[3] = static_cast<_Float16>(x.w * kLog2e);
        h[4] = static_cast<_Float16>(y.x * kLog2e); h[5] = static_cast<_Float16>(y.y * kLog2e);
        h[6] = static_cast<_Float16>(y.z * kLog2e); h[7] = static_cast<_Float16>(y.w * kLog2e);
        wb[nt][ks] = h;
      } else {
        wb[nt][ks] = *reinterpret_cast<const f16x8*>(a.W16 + (64 * fw + 16 * nt + l16) * WROW +
                                                     32 * ks + 8 * g);
      }
    }
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) cref[nt] = 0.f;

  // Slot r of the ring holds tiles r, r + 6, ...; the slot index is a
  // compile-time constant at every use (the step loop is unrolled six
  // times), so the per-lane LDS addresses below are formed once and the
  // slot's offset is the instructions' immediate.
  using I0 = std::integral_constant<int, 0>;
  const uint32_t ring_a = static_cast<uint32_t>(tg * NSLOT * SLOT_BYTES);   // offset of `ring`
  // Byte offset of the slot holding tile R: a compile-time constant for the
  // unrolled fast loop, computed for the slow loop and the ReLU features'
  // loop (not unrolled: their register allocation does not fit six copies).
  auto soff = [](auto R) {
    if constexpr (std::is_integral_v<decltype(R)>) return (R % NSLOT) * SLOT_BYTES;
    else return decltype(R)::value * SLOT_BYTES;
  };
  // This wave's quarter of tile i (slot R) of the group (two DMA
  // instructions): slot unit u = 128 fw + 64 j + lane, units 0..255 the K rows
  // and 256..511 the V rows; unit u of a row holds the row's global unit
  // (u % 8) ^ (row % 8).  Rows past the split read zero.
  auto dma_part = [&](auto R, int i, int j) {
    const int tb = tile_base(i);
    const int uu = (128 * fw + 64 * j + lane) & 255, row = uu >> 3, gu = (uu & 7) ^ (row & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc_kv, (lds_ptr)(ring + soff(R) + 16 * (128 * fw + 64 * j)), 16,
        ((tb + row) * FD + 8 * gu) * 2, 0, 0, 0);
  };
  // K rows 8 fw .. + 7 of tile i (slot R) to fp16 in place (lane: row
  // 8 fw + lane / 8, 16-byte unit lane % 8) and their norm terms (8 lanes per
  // row).
  const int crow = 8 * fw + (lane >> 3);
  const uint32_t cvt_a = ring_a + crow * 128 + (lane & 7) * 16;
  const uint32_t cvt_nb = ring_a + SLOT_NB + crow * 4;
  auto convert = [&](auto R, int i) {
    const int off = soff(R);
    auto* const p = lds_at<u32x4>(cvt_a + off);
    const u32x4 x = *p;
    const uint32_t w0 = x[0], w1 = x[1], w2 = x[2], w3 = x[3];
    float ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0),
                                               __builtin_bit_cast(bf16x2, w0), 0.f, false);
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1),
                                         __builtin_bit_cast(bf16x2, w1), ss, false);
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2),
                                         __builtin_bit_cast(bf16x2, w2), ss, false);
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3),
                                         __builtin_bit_cast(bf16x2, w3), ss, false);
    ss = group_sum<8>(ss);
    *p = u32x4{bf16x2_to_f16x2(w0), bf16x2_to_f16x2(w1), bf16x2_to_f16x2(w2), bf16x2_to_f16x2(w3)};
    const int tb = tile_base(i);
    if ((lane & 7) == 0) *lds_at<float>(cvt_nb + off) = tb + crow < n ? nscale * ss : -INFINITY;
  };
  // Operand addresses of the projection (token 16 mt + l16, dims 32 ks +
  // 8 g .. + 7, fp16) and of its C input (rows 16 mt + 4 g .. + 3).
  uint32_t kop_a[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row = 16 * mt + l16, c = 4 * ks + g;
      kop_a[mt][ks] = ring_a + row * 128 + ((c ^ (row & 7)) * 16);
    }
  const uint32_t nq_a = ring_a + SLOT_NB + 16 * g;
  // Transposing-read addresses of the contraction's V^T operand (value
  // column 16 mv + l16; read r of a pair adds 16 rows, 2048 bytes).
  uint32_t tr_a[4];
  {
    const int row = 4 * g + (l16 >> 2);
#pragma unroll
    for (int mv = 0; mv < 4; ++mv)
      tr_a[mv] = lds_addr0() + ring_a + KT_BYTES + row * 128 +
                 (((2 * mv + ((l16 & 3) >> 1)) ^ (row & 7)) * 16) + (l16 & 1) * 8;
  }
  using SArr = f32x4[2][4];
  // S for tile i: fp16 operands (token 16 mt + l16, dims 32 ks + 8 g .. + 7)
  // and the C input -n (rows 16 mt + 4 g .. + 3) from the slot.
  auto proj = [&](auto R, SArr& S) {
    const int off = soff(R);
    f16x8 ka[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ka[mt][ks] = *lds_at<const f16x8>(kop_a[mt][ks] + off);
    f32x4 nq[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) nq[mt] = *lds_at<const f32x4>(nq_a + off + 64 * mt);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if constexpr (SLOW) S[mt][nt] = mma_f16(ka[mt][0], wb[nt][0], nq[mt] - cref[nt]);
        else S[mt][nt] = mma_f16(ka[mt][0], wb[nt][0], nq[mt]);
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[mt][nt] = mma_f16(ka[mt][1], wb[nt][1], S[mt][nt]);
  };
  auto features = [&](const SArr& S, bf16x8 (&kb)[4]) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        p[q] = pack_bf16(feature<RELU>(S[0][nt][2 * q]), feature<RELU>(S[0][nt][2 * q + 1]));
        p[2 + q] = pack_bf16(feature<RELU>(S[1][nt][2 * q]), feature<RELU>(S[1][nt][2 * q + 1]));
      }
      kb[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
    }
  };
  // (slow) some feature reached 2, or is not finite
  auto overflow = [&](const bf16x8 (&kb)[4]) {
    uint32_t o = 0;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint4 w = __builtin_bit_cast(uint4, kb[nt]);
      o |= w.x | w.y | w.z | w.w;
    }
    return __ballot((o & 0x40004000u) != 0) != 0;
  };
  // (slow) reference update from the tile's exact per-feature maximum: set
  // on the wave's first tile kKeyBias above it, later raised where exceeded
  // (the accumulators and the projected tile move along).
  auto rebase = [&](SArr& S, bool first) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float x = max3(S[0][nt][0], S[0][nt][1], S[0][nt][2]);
      const float y = max3(S[0][nt][3], S[1][nt][0], S[1][nt][1]);
      const float tm = colmax4(max3(x, y, fmaxf(S[1][nt][2], S[1][nt][3])));
      const float dlt = (tm == -INFINITY) ? 0.f
                                          : (first ? tm + kKeyBiasF : fmaxf(tm + kKeyBiasF, 0.f));
      if (!first) {
        const float f = fast_exp2(-dlt);
#pragma unroll
        for (int i = 0; i < 5; ++i) acc[i][nt] *= f;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) S[mt][nt] -= dlt;
      cref[nt] += dlt;
    }
  };
  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = static_cast<__bf16>(1.0f);
  // [V | 1]^T K~ for tile i: operand row = value column 16 mv + l16,
  // positions 8 g + 0..3 / 4..7 = tokens 4 g + 0..3 / 16 + 4 g + 0..3 (read
  // r: lane l16 of the 16-lane group g addresses row 16 r + 4 g + l16/4,
  // columns 16 mv + 4 (l16 % 4) .. + 3, and receives column 16 mv + l16 of
  // rows 16 r + 4 g .. + 3).
  auto contract_half = [&](auto R, const bf16x8 (&kb)[4], int half) {
    // The four transposing reads of the half are issued together and waited
    // for in the same statement (the compiler would otherwise wait for every
    // LDS DMA in flight before each of them; this tile's DMA has landed).
    uint64_t h[4];
    if constexpr (std::is_integral_v<decltype(R)>) {
      const uint32_t o = static_cast<uint32_t>(soff(R));
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
          "ds_read_b64_tr_b16 %2, %5\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:2048\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
          : "v"(tr_a[2 * half] + o), "v"(tr_a[2 * half + 1] + o)
          : "memory");
    } else {
      constexpr int off = decltype(R)::value * SLOT_BYTES;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
          "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
          "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
          : "v"(tr_a[2 * half]), "v"(tr_a[2 * half + 1]), "n"(off), "n"(off + 2048)
          : "memory");
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int mv = 2 * half + u;
      const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(static_cast<uint32_t>(h[2 * u]),
                                                              static_cast<uint32_t>(h[2 * u] >> 32),
                                                              static_cast<uint32_t>(h[2 * u + 1]),
                                                              static_cast<uint32_t>(h[2 * u + 1] >> 32)));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mv][nt] = mma_bf16(va, kb[nt], acc[mv][nt]);
    }
    if (half == 1) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[4][nt] = mma_bf16(ones, kb[nt], acc[4][nt]);
    }
  };

  // Prologue: tiles 0..4 in flight; tile 0 converted once it has landed
  // everywhere (this wave's tiles 1..4 may be in flight: eight operations),
  // tile 1 likewise (six), then tile 0 projected and its features formed.
  // DMAs past the group's last tile read zeros, so every step issues the
  // same number of operations.
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  dma_part(I0{}, 0, 0); dma_part(I0{}, 0, 1);
  dma_part(I1{}, 1, 0); dma_part(I1{}, 1, 1);
  dma_part(I2{}, 2, 0); dma_part(I2{}, 2, 1);
  dma_part(I3{}, 3, 0); dma_part(I3{}, 3, 1);
  dma_part(I4{}, 4, 0); dma_part(I4{}, 4, 1);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  lds_barrier();
  convert(I0{}, 0);
  asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  lds_barrier();
  convert(I1{}, 1);
  bf16x8 kbA[4], kbB[4];
  {
    SArr S;
    proj(I0{}, S);
    if constexpr (SLOW) rebase(S, true);
    features(S, kbA);
  }
  // Step i (tile i in slot R = i % 6): tile i + 2 has landed (this wave's
  // tiles i + 3, i + 4 may be in flight) and tile i + 1 is converted
  // everywhere; every wave is done with tile i - 1, whose slot takes tile
  // i + 5.  The tile's two DMA instructions go between the matrix work
  // (after the projection, halfway through the contraction) rather than in
  // a burst after the barrier: an instruction that finds the memory
  // pipeline's queue full holds up its wave.
  auto step = [&](auto R, int i, const bf16x8 (&kcur)[4], bf16x8 (&knext)[4]) {
    auto r1 = [&]() {
      if constexpr (std::is_integral_v<decltype(R)>) return i + 1;
      else return std::integral_constant<int, (decltype(R)::value + 1) % NSLOT>{};
    }();
    auto r2 = [&]() {
      if constexpr (std::is_integral_v<decltype(R)>) return i + 2;
      else return std::integral_constant<int, (decltype(R)::value + 2) % NSLOT>{};
    }();
    auto r5 = [&]() {
      if constexpr (std::is_integral_v<decltype(R)>) return i + 5;
      else return std::integral_constant<int, (decltype(R)::value + 5) % NSLOT>{};
    }();
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    lds_barrier();
    convert(r2, i + 2);
    SArr S;
    proj(r1, S);
    dma_part(r5, i + 5, 0);
    contract_half(R, kcur, 0);
    dma_part(r5, i + 5, 1);
    contract_half(R, kcur, 1);
    features(S, knext);
    if constexpr (SLOW) {
      if (__builtin_expect(overflow(knext), 0)) {
        rebase(S, false);
        features(S, knext);
      }
    }
  };
  static_assert(NSLOT == 6, "the fast step loop is unrolled once around the ring");
  if constexpr (SLOW || RELU) {
    for (int i = 0; i < nsteps; i += 2) {
      step(i, i, kbA, kbB);
      if (i + 1 >= nsteps) break;
      step(i + 1, i + 1, kbB, kbA);
    }
  } else for (int i = 0; i < nsteps; i += 6) {
    step(I0{}, i, kbA, kbB);
    if (i + 1 >= nsteps) break;
    step(I1{}, i + 1, kbB, kbA);
    if (i + 2 >= nsteps) break;
    step(I2{}, i + 2, kbA, kbB);
    if (i + 3 >= nsteps) break;
    step(I3{}, i + 3, kbB, kbA);
    if (i + 4 >= nsteps) break;
    step(I4{}, i + 4, kbA, kbB);
    if (i + 5 >= nsteps) break;
    step(I5{}, i + 5, kbB, kbA);
  }
  // (the DMAs issued past the group's last tile land before the LDS is reused)
  vm_drain();
  // A group that saw no token carries no reference.
  if (SEP ? ntl == 0 : tg >= ntl) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) cref[nt] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Key item (head bh, split s, tokens [s seg, min(L, (s + 1) seg))): the pass
// and the merge of the two token groups (the second group's sums into the
// first's, rescaled to the larger reference); if the sums are not finite, or
// some feature's ones-column sum fell below 2^-100 (its features underflow
// without a reference), both again with references.  The first group's waves
// write the partial [65][256] fp32 and its references with device-scope
// stores; the work-group waits for them and arrives at its head.
// ---------------------------------------------------------------------------
template <bool RELU>
__device__ __forceinline__ void key_item(const Args& a, int bh, int s, unsigned* snapq,
                                         unsigned (&snap)[NXCD]) {
  unsigned* const bc = bcast();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6), tg = wave / NFW, fw = wave % NFW;
  const int l16 = lane & 15, g = lane >> 4;
  const int t0 = s * a.seg, t1 = min(a.L, t0 + a.seg);
  f32x4 acc[5][4];
  float cref[4];
  for (int pass = 0; pass < 2; ++pass) {
    const bool slow = pass == 1;
    if (slow) key_pass<RELU, true>(a, bh, t0, t1, acc, cref);
    else key_pass<RELU, false>(a, bh, t0, t1, acc, cref);
    lds_barrier();   // the ring is read: the merge slots take its bytes
    if (tg == 1) {
      f32x4* slot = reinterpret_cast<f32x4*>(g_smem + fw * MERGE_SLOT) + lane;
#pragma unroll
      for (int mv = 0; mv < 5; ++mv)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) slot[(mv * 4 + nt) * 64] = acc[mv][nt];
      slot[20 * 64] = f32x4{cref[0], cref[1], cref[2], cref[3]};
    }
    lds_barrier();
    bool bad = false;
    if (tg == 0) {
      const f32x4* slot = reinterpret_cast<const f32x4*>(g_smem + fw * MERGE_SLOT) + lane;
      const f32x4 co = slot[20 * 64];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float cn = fmaxf(cref[nt], co[nt]);
        const float x = rescale(cref[nt], cn), y = rescale(co[nt], cn);
#pragma unroll
        for (int mv = 0; mv < 5; ++mv) acc[mv][nt] = acc[mv][nt] * x + slot[(mv * 4 + nt) * 64] * y;
        cref[nt] = cn;
      }
      if (!RELU && !slow) {
#pragma unroll
        for (int i = 0; i < 5; ++i)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) bad |= !__builtin_isfinite(acc[i][nt][v]);
        if (g == 0) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) bad |= !(acc[4][nt][0] >= 0x1p-100f);
        }
      }
    }
    if (RELU || slow) break;
    if (tid == 0) bc[0] = 0u;
    lds_barrier();
    if (bad) bc[0] = 1u;
    lds_barrier();
    if (bc[0] == 0u) break;
  }
  if (tg == 0) {
    // Partial rows 16 mv + 4 g + v (row 64: the ones column), features
    // 64 fw + 16 nt + l16; references of those features.
    const size_t item = static_cast<size_t>(bh) * a.nsplit + s;
    const __amdgpu_buffer_rsrc_t rt = buffer_rsrc(a.T + item * PROWS * FM, PROWS * FM * 4);
#pragma unroll
    for (int mv = 0; mv < 5; ++mv)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * mv + 4 * g + v;
        if (row < PROWS) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            store4_sc1(rt, (row * FM + 64 * fw + 16 * nt + l16) * 4, acc[mv][nt][v]);
        }
      }
    if (g == 0) {
      const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.cs + item * FM, FM * 4);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) store4_sc1(rc, (64 * fw + 16 * nt + l16) * 4, cref[nt]);
    }
  }
  // (the queue-head snapshot is read while the stores drain)
  if (tid == 0) take_snapshot(snapq, snap);
  vm_drain();
  lds_barrier();   // every wave's stores have completed
  if (tid == 0)
    __hip_atomic_fetch_add(a.ctrl + Ctrl::arrive(bh), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Query item: block qb of head bh, tokens [qb QB, min(L, (qb+1) QB)), in
// 32-token tiles (wave w takes tiles w, w + 8, ...).  LDS: W' [256][72]
// fp16, the state [80][264] bf16 (query operand order), the references c
// [256] fp32.  The state is the sum of the head's partials, each rescaled to
// the per-feature maximum c of their references.  Per tile, for each
// 64-feature chunk: S^T = W' Q^T + C, Q~ = exp2(S^T) in bf16, and
// [KV | z]^T Q~^T accumulated in fp32; the next chunk is projected while the
// current one is applied.  O = num / den.  C is the query's norm term
// -|q|^2 log2(e) / 2 (a per-row shift that cancels in D^-1 and bounds the
// exponent by |w|^2 log2(e) / 2); a tile whose denominators leave
// [2^-100, 2^100], and every tile of a head whose state carries references,
// takes instead C = c_r - M with M its exact row maximum of s + c_r.
// ---------------------------------------------------------------------------
using Qraw = uint4[2][2];
using Qop = f16x8[2][2];
using QS = f32x4[4][2];
using QFeat = bf16x8[2][2];   // [kb][nt]: lane = token, 8 features (perm_of)
using QAcc = f32x4[5][2];

// Position of feature f in the state's row (query operand order): within
// each 32-feature block, feature 4 q + i at 8 q + i and 16 + 4 q + i at
// 8 q + 4 + i.
__device__ inline int state_pos(int f) {
  const int j = f & 31;
  return (f & ~31) + (j < 16 ? 8 * (j >> 2) + (j & 3) : 8 * ((j - 16) >> 2) + 4 + (j & 3));
}

template <bool RELU>
__device__ __forceinline__ void query_item(const Args& a, int bh, int qb, unsigned* snapq,
                                           unsigned (&snap)[NXCD]) {
  unsigned char* const smem = g_smem;
  unsigned* const bc = bcast();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  _Float16* const Wl = reinterpret_cast<_Float16*>(smem);
  uint16_t* const Kzl = reinterpret_cast<uint16_t*>(smem + QW_BYTES);
  float* const cl = reinterpret_cast<float*>(smem + QW_BYTES + QK_BYTES);
  float* const scl = reinterpret_cast<float*>(smem + QW_BYTES + QK_BYTES + QC_BYTES);
  const int L = a.L, nsplit = a.nsplit;
  const size_t base = static_cast<size_t>(bh) * L * FD;
  const int q0 = qb * a.QB, q1 = min(L, q0 + a.QB);

  // W' (written by the previous launch) straight into LDS.
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.W16);
    uint4* dst = reinterpret_cast<uint4*>(Wl);
    constexpr int n16 = FM * WROW / 8;
    for (int j = wave; 64 * j < n16; j += NW)
      if (64 * j + lane < n16) lds_dma16(src + 64 * j + lane, dst + 64 * j);
  }
  // The wave's first tile of Q, loaded while the head's state is awaited.
  const uint16_t* const Qh = a.Q + base;
  uint16_t* const Oh = a.O + base;
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qh, q1 * FD * 2);
  const int tstep = NW * QTILE;
  const int tt0 = q0 + wave * QTILE;
  const int ntile = tt0 < q1 ? (q1 - tt0 + tstep - 1) / tstep : 0;
  auto q_load = [&](int tt, Qraw& raw) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        raw[nt][ks] = buffer_load16(rq, ((tt + 16 * nt + l16) * FD + 32 * ks + 8 * g) * 2);
  };
  Qraw raw;
  q_load(tt0, raw);

  // Wait until every split of the head has written its partial.
  if (tid == 0) {
    unsigned r = 0, spins = 0;
    while ((r = load_sc1(a.ctrl + Ctrl::arrive(bh))) < static_cast<unsigned>(nsplit)) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins >= kSpinLimit) {
        store_sc1(a.ctrl + Ctrl::TIMEOUT, 1u);
        break;
      }
    }
    bc[0] = r >= static_cast<unsigned>(nsplit) ? 1u : 0u;
    bc[1] = 0u;
  }
  // (LDS only: W' and the first Q tile stay in flight)
  lds_barrier();
  const unsigned ready = bc[0];
  if (ready == 0u) {
    // (the wait gave up: the output of this block is marked invalid)
    vm_drain();
    for (int i = tid; i < (q1 - q0) * FD; i += FNT) Oh[static_cast<size_t>(q0) * FD + i] = 0x7FC0u;
    __syncthreads();
    return;
  }
  // The state: partials (device-scope loads, issued first), the per-feature
  // maximum c of their references and each split's scale 2^(c_s - c), then
  // the rescaled sum in bf16.  Thread t sums the 4-feature units t + 512 k
  // of the [65][256] partial (splits past the head's read zero, scale 0).
  {
    const size_t item0 = static_cast<size_t>(bh) * nsplit;
    const __amdgpu_buffer_rsrc_t rt =
        buffer_rsrc(a.T + item0 * PROWS * FM, nsplit * PROWS * FM * 4);
    constexpr int NU = PROWS * FM / 4;           // 4160 units
    constexpr int NK = (NU + FNT - 1) / FNT;     // 9 per thread at most
    constexpr int NKA = 5;                       // first batch
    uint4 x[NKA][NSPLIT];
#pragma unroll
    for (int k = 0; k < NKA; ++k)
#pragma unroll
      for (int s = 0; s < NSPLIT; ++s)
        x[k][s] = load16_sc1(rt, ((s * PROWS * FM) + 4 * (tid + FNT * k)) * 4);
    if (tid < FM) {
      const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.cs + item0 * FM, nsplit * FM * 4);
      float c[NSPLIT];
#pragma unroll
      for (int s = 0; s < NSPLIT; ++s) c[s] = load4_sc1(rc, (s * FM + tid) * 4);
      float cn = -INFINITY;
#pragma unroll
      for (int s = 0; s < NSPLIT; ++s)
        if (s < nsplit) cn = fmaxf(cn, c[s]);
#pragma unroll
      for (int s = 0; s < NSPLIT; ++s) scl[s * FM + tid] = s < nsplit ? rescale(c[s], cn) : 0.f;
      cl[tid] = cn;
      if (cn != 0.f) bc[1] = 1u;   // some reference is not 0
    }
    lds_barrier();
    auto combine = [&](int u, const uint4 (&xs)[NSPLIT]) {
      const int row = u / (FM / 4), f = 4 * (u % (FM / 4));
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int s = 0; s < NSPLIT; ++s) {
        const float4 w = *reinterpret_cast<const float4*>(&scl[s * FM + f]);
        const uint4 v = xs[s];
        sum.x = fmaf(w.x, __uint_as_float(v.x), sum.x);
        sum.y = fmaf(w.y, __uint_as_float(v.y), sum.y);
        sum.z = fmaf(w.z, __uint_as_float(v.z), sum.z);
        sum.w = fmaf(w.w, __uint_as_float(v.w), sum.w);
      }
      *reinterpret_cast<uint2*>(&Kzl[row * KZROW + state_pos(f)]) =
          make_uint2(pack_bf16(sum.x, sum.y), pack_bf16(sum.z, sum.w));
    };
#pragma unroll
    for (int k = 0; k < NKA; ++k) {
      const int u = tid + FNT * k;
      if (u < NU) combine(u, x[k]);
    }
    uint4 y[NK - NKA][NSPLIT];
#pragma unroll
    for (int k = NKA; k < NK; ++k)
#pragma unroll
      for (int s = 0; s < NSPLIT; ++s)
        y[k - NKA][s] = load16_sc1(rt, ((s * PROWS * FM) + 4 * (tid + FNT * k)) * 4);
#pragma unroll
    for (int k = NKA; k < NK; ++k) {
      const int u = tid + FNT * k;
      if (u < NU) combine(u, y[k - NKA]);
    }
    // rows 65..79 of the operand are zero
    for (int i = tid; i < (KZROWS - PROWS) * FM / 8; i += FNT) {
      const int row = PROWS + i / (FM / 8), c8 = 8 * (i % (FM / 8));
      *reinterpret_cast<uint4*>(&Kzl[row * KZROW + c8]) = make_uint4(0, 0, 0, 0);
    }
  }
  vm_drain();   // W' has landed
  lds_barrier();
  const bool refs = bc[1] != 0u;
  if (tid == 0) take_snapshot(snapq, snap);

  // S^T + C for chunk ch: rows features 64 ch + 16 mt + 4 g + v, column
  // token.  Fast form: C = cq[nt], the per-token norm term, as the matrix
  // instruction's C operand; slow form: C = c_r + cq[nt].
  auto proj = [&](auto SLOWC, int ch, const Qop& qop, const f32x4 (&cq)[2], QS& S) {
    constexpr bool SL = decltype(SLOWC)::value;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 wa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        wa[mt] = *reinterpret_cast<const f16x8*>(&Wl[(64 * ch + 16 * mt + l16) * WROW + 32 * ks + 8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (ks == 0) {
          if constexpr (SL) {
            const f32x4 crow = *reinterpret_cast<const f32x4*>(&cl[64 * ch + 16 * mt + 4 * g]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mma_f16(wa[mt], qop[nt][0], crow + cq[nt]);
          } else {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mma_f16(wa[mt], qop[nt][0], cq[nt]);
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mma_f16(wa[mt], qop[nt][1], S[mt][nt]);
        }
      }
    }
  };
  auto features = [&](const QS& S, QFeat& qt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          p[q] = pack_bf16(feature<RELU>(S[2 * kb][nt][2 * q]), feature<RELU>(S[2 * kb][nt][2 * q + 1]));
          p[2 + q] = pack_bf16(feature<RELU>(S[2 * kb + 1][nt][2 * q]),
                               feature<RELU>(S[2 * kb + 1][nt][2 * q + 1]));
        }
        qt[kb][nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
      }
  };
  auto apply = [&](int ch, const QFeat& qt, QAcc& acc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kcol = 64 * ch + 32 * kb + 8 * g;
#pragma unroll
      for (int mv = 0; mv < 5; ++mv) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kzl[(16 * mv + l16) * KZROW + kcol]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mv][nt] = mma_bf16(ka, qt[kb][nt], acc[mv][nt]);
      }
    }
  };
  // The four chunks of a tile: chunk ch + 1 projected while chunk ch is
  // applied.
  auto tile = [&](auto SLOWC, const Qop& qop, const f32x4 (&cq)[2], QAcc& acc) {
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    QFeat FA, FB;
    {
      QS S;
      proj(SLOWC, 0, qop, cq, S);
      features(S, FA);
    }
    auto regular = [&](const int ch, const QFeat& Fcur, QFeat& Fnext) {
      __builtin_amdgcn_sched_barrier(0);
      QS S;
      proj(SLOWC, ch + 1, qop, cq, S);
      apply(ch, Fcur, acc);
      features(S, Fnext);
      interleave_mfma_valu<16, 20, 3>();
    };
    regular(0, FA, FB);
    regular(1, FB, FA);
    regular(2, FA, FB);
    __builtin_amdgcn_sched_barrier(0);
    apply(3, FB, acc);
  };
  // The slow form's C offset: minus the exact row maximum of s + c_r.
  auto row_max = [&](const Qop& qop, f32x4 (&cq)[2]) {
    float mx[2] = {-INFINITY, -INFINITY};
    const f32x4 zc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int ch = 0; ch < FNCH; ++ch) {
      QS S;
      proj(std::true_type{}, ch, qop, zc, S);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          mx[nt] = fmaxf(mx[nt], max3(S[mt][nt][0], S[mt][nt][1], fmaxf(S[mt][nt][2], S[mt][nt][3])));
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float m = -colmax4(mx[nt]);
      cq[nt] = f32x4{m, m, m, m};
    }
  };
  // den of token column l16 (row 64: tile 4, row 0, held by lanes g = 0).
  auto den_of = [&](const QAcc& acc, int nt) { return __shfl(acc[4][nt][0], l16, 64); };
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(Oh, q1 * FD * 2);
  auto store = [&](const QAcc& acc, int tt) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float inv = 1.0f / den_of(acc, nt);
      const int tok = tt + 16 * nt + l16;
#pragma unroll
      for (int mv = 0; mv < 4; ++mv) {
        const uint32_t x = pack_bf16(acc[mv][nt][0] * inv, acc[mv][nt][1] * inv);
        const uint32_t y = pack_bf16(acc[mv][nt][2] * inv, acc[mv][nt][3] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{x, y}, ro, (tok * FD + 4 * g + 16 * mv) * 2, 0, 0);
      }
    }
  };

  for (int ti = 0; ti < ntile; ++ti) {
    const int tt = tt0 + ti * tstep;
    // Q^T operands in fp16 (token 16 nt + l16, dims 32 ks + 8 g .. + 7) and
    // the per-token norm term -|q|^2 log2(e) / 2.
    Qop qop;
    f32x4 cq[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 x = raw[nt][ks];
        if constexpr (!RELU) {
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.x),
                                               __builtin_bit_cast(bf16x2, x.x), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.y),
                                               __builtin_bit_cast(bf16x2, x.y), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.z),
                                               __builtin_bit_cast(bf16x2, x.z), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.w),
                                               __builtin_bit_cast(bf16x2, x.w), ss, false);
        }
        qop[nt][ks] = __builtin_bit_cast(
            f16x8, make_uint4(bf16x2_to_f16x2(x.x), bf16x2_to_f16x2(x.y), bf16x2_to_f16x2(x.z),
                              bf16x2_to_f16x2(x.w)));
      }
      const float nq = RELU ? 0.f : -0.5f * kLog2e * colsum4(ss);
      cq[nt] = f32x4{nq, nq, nq, nq};
    }
    if (ti + 1 < ntile) q_load(tt + tstep, raw);
    QAcc acc;
    bool slow = !RELU && refs;
    if (!slow) {
      tile(std::false_type{}, qop, cq, acc);
      if constexpr (!RELU) {
        bool bad = false;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float den = den_of(acc, nt);
          bad |= (tt + 16 * nt + l16 < q1) && !(den >= 0x1p-100f && den <= 0x1p100f);
        }
        slow = __ballot(bad) != 0;
      }
    }
    if constexpr (!RELU) {
      if (slow) {
        row_max(qop, cq);
        tile(std::true_type{}, qop, cq, acc);
      }
    }
    store(acc, tt);
  }
  lds_barrier();   // every wave is done with the LDS (the O stores may still drain)
}

// ---------------------------------------------------------------------------
// fused: the persistent kernel.  Heads are dealt to the eight dies in turn;
// die x's key queue holds items v = (head index on the die) nsplit + split
// and its query queue v = (head index) nqb + block, both head-major, so that
// a head's splits are claimed together and its query blocks soon after.  A
// work-group claims from its own die's queues (the partials a query item
// sums were mostly written by work-groups of its die: they are fresh in the
// die's L2), and once those are empty from any die with items left; no
// items left anywhere ends the phase.  Key items first, then query items.
// Thread 0 claims and the item goes through LDS.  It claims a key item and
// a query item at the start (the query claim is held until every key queue
// is empty), and while each item runs it reads every die's queue heads: a
// queue seen empty stays empty, so the next claim (an atomic, which the
// work-groups of a die would otherwise queue up on) is made only where
// items may be left, and the phase ends without a claim once all are seen
// empty.
// ---------------------------------------------------------------------------
__device__ inline unsigned die_items(int BH, int x, int per_head) {
  return static_cast<unsigned>(x < BH ? (BH - x + NXCD - 1) / NXCD * per_head : 0);
}

// Thread 0: an item of the queues at word `qbase` given the own-die claim
// `own` and a snapshot `c` of every die's queue head (zeros: not taken):
// die * 2^24 + index, or -1 when no die has items left.
__device__ inline int pick_item(unsigned* ctrl, int qbase, int per_head, int BH, int my,
                                unsigned own, unsigned (&c)[NXCD]) {
  if (own < die_items(BH, my, per_head)) return (my << 24) | static_cast<int>(own);
  for (;;) {
    int pick = -1;
#pragma unroll
    for (int k = 1; k < NXCD; ++k) {
      const int x = (my + k) % NXCD;
      if (pick < 0 && c[x] < die_items(BH, x, per_head)) pick = x;
    }
    if (pick < 0) return -1;
    const unsigned v = __hip_atomic_fetch_add(ctrl + qbase + Ctrl::LINE * pick, 1u,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v < die_items(BH, pick, per_head)) return (pick << 24) | static_cast<int>(v);
    // (other work-groups took that die's last items: the counts only grow,
    // so this loop ends)
#pragma unroll
    for (int x = 0; x < NXCD; ++x) c[x] = load_sc1(ctrl + qbase + Ctrl::LINE * x);
  }
}

template <bool RELU>
__global__ __launch_bounds__(FNT, 1) void fused(Args a) {
  unsigned* const bc = bcast();
  const bool lead = threadIdx.x == 0;
  // (this work-group's die: hardware register XCC_ID, bits 3:0)
  const int my = static_cast<int>(__builtin_amdgcn_s_getreg(20 | (3 << 11))) % NXCD;
  unsigned* const kq = a.ctrl + Ctrl::kq(0);
  unsigned* const qq = a.ctrl + Ctrl::qq(0);
  const unsigned kmine = die_items(a.BH, my, a.nsplit), qmine = die_items(a.BH, my, a.nqb);
  unsigned own = 0, qown = 0;
  unsigned c[NXCD];
  if (lead) {
    // A key item and a query item claimed at once (the query claim is used
    // once every key queue is empty).
    own = __hip_atomic_fetch_add(kq + Ctrl::LINE * my, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    qown = __hip_atomic_fetch_add(qq + Ctrl::LINE * my, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int x = 0; x < NXCD; ++x) c[x] = 0u;
  }
  for (;;) {
    if (lead) bc[8] = static_cast<unsigned>(pick_item(a.ctrl, Ctrl::kq(0), a.nsplit, a.BH, my, own, c));
    lds_barrier();
    const int it = static_cast<int>(bc[8]);
    lds_barrier();
    if (it < 0) break;
    const int x = it >> 24, v = it & 0xFFFFFF;
    key_item<RELU>(a, x + NXCD * (v / a.nsplit), v % a.nsplit, kq, c);
    // (the snapshot taken during the item says whether the own queue can
    // still have items: only then is another claimed)
    if (lead)
      own = c[my] < kmine ? __hip_atomic_fetch_add(kq + Ctrl::LINE * my, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                          : kmine;
  }
  if (lead) {
#pragma unroll
    for (int x = 0; x < NXCD; ++x) c[x] = 0u;
  }
  for (;;) {
    if (lead) bc[8] = static_cast<unsigned>(pick_item(a.ctrl, Ctrl::qq(0), a.nqb, a.BH, my, qown, c));
    lds_barrier();
    const int it = static_cast<int>(bc[8]);
    lds_barrier();
    if (it < 0) break;
    const int x = it >> 24, v = it & 0xFFFFFF;
    query_item<RELU>(a, x + NXCD * (v / a.nqb), v % a.nqb, qq, c);
    if (lead)
      qown = c[my] < qmine ? __hip_atomic_fetch_add(qq + Ctrl::LINE * my, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                           : qmine;
  }
}

// ---------------------------------------------------------------------------
// ckey: the key states of the causal form's segments (every segment but the
// last; the prefix-sum form needs, for each segment, the sum over the keys
// of the segments before it).  Work-group (head bh, pair pr) takes segments
// 2 pr and 2 pr + 1, one per token group, each group over its own segment
// with the key pass above: a group's sums are its segment's state, so no
// merge.  The state [(K')^T V | (K')^T 1] of segment s goes to
// T[bh][s][65][256] in fp32 with its per-feature references in
// cs[bh][s][256] (log2 units), the layout the prefix kernel reads.  A group
// whose sums are not finite, or whose ones-column sum fell below 2^-100,
// makes the work-group redo both segments with per-feature references.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(FNT, 1) void ckey(Args a, int npair, int nneed) {
  unsigned* const bc = bcast();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6), tg = wave / NFW, fw = wave % NFW;
  const int l16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / npair, pr = blockIdx.x - bh * npair;
  const int s = 2 * pr + tg;
  const bool has = s < nneed;
  const int t0 = has ? s * a.seg : 0, t1 = has ? min(a.L, t0 + a.seg) : 0;
  f32x4 acc[5][4];
  float cref[4];
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) key_pass<false, true, true>(a, bh, t0, t1, acc, cref, a.seg);
    else key_pass<false, false, true>(a, bh, t0, t1, acc, cref, a.seg);
    if (pass == 1) break;
    bool bad = false;
    if (has) {
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) bad |= !__builtin_isfinite(acc[i][nt][v]);
      if (g == 0) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bad |= !(acc[4][nt][0] >= 0x1p-100f);
      }
    }
    // (the barriers also order every wave's last ring reads before a redo's
    // first DMAs)
    if (tid == 0) bc[0] = 0u;
    lds_barrier();
    if (bad) bc[0] = 1u;
    lds_barrier();
    if (bc[0] == 0u) break;
  }
  if (!has) return;
  const size_t item = static_cast<size_t>(bh) * a.nsplit + s;
  float* const T = a.T + item * PROWS * FM;
#pragma unroll
  for (int mv = 0; mv < 5; ++mv)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * mv + 4 * g + v;
      if (row < PROWS) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) T[row * FM + 64 * fw + 16 * nt + l16] = acc[mv][nt][v];
      }
    }
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) a.cs[item * FM + 64 * fw + 16 * nt + l16] = cref[nt];
  }
}

}  // namespace

bool fused_bidir_supported(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype) {
  (void)L;
  return dtype == FAVOR_BF16 && d == FD && m == FM && static_cast<int64_t>(B) * H >= 64;
}

void fused_bidir_layout(Plan* p, int cus) {
  const int BH = p->BH, L = p->L;
  // Key items: up to four splits per head, each a whole number of 32-token
  // tiles and at least 256 tokens (every split holds at least one token).
  int64_t seg = (static_cast<int64_t>(L) + NSPLIT - 1) / NSPLIT;
  seg = (seg + FTT - 1) / FTT * FTT;
  if (seg < 256) seg = 256;
  p->seg = static_cast<int32_t>(seg);
  p->nseg = static_cast<int32_t>((L + seg - 1) / seg);
  // Query blocks: about one query item per compute unit, a multiple of 256
  // tokens (one 32-token tile per wave).
  const int64_t want = (static_cast<int64_t>(L) * BH + cus - 1) / cus;
  int64_t qb = (want + 255) / 256 * 256;
  qb = qb < 256 ? 256 : qb;
  p->qblk = static_cast<int32_t>(qb > L ? (static_cast<int64_t>(L) + 255) / 256 * 256 : qb);
}

hipError_t fused_bidir_forward(const Plan& p, const void* Q, const void* K, const void* V,
                               const float* W, void* O, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  Args a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = static_cast<uint16_t*>(O);
  a.W16 = reinterpret_cast<const _Float16*>(w + p.off_cP);
  a.T = reinterpret_cast<float*>(w + p.off_T);
  a.cs = reinterpret_cast<float*>(w + p.off_cseg);
  a.ctrl = reinterpret_cast<unsigned*>(w + p.off_ctrl);
  a.L = p.L;
  a.BH = p.BH;
  a.nsplit = p.nseg;
  a.seg = p.seg;
  a.QB = p.qblk;
  a.nqb = (p.L + p.qblk - 1) / p.qblk;
  a.knorm = p.knorm;
  const int nctrl = static_cast<int>(fused_ctrl_words(p.BH));
  timing_before(st);
  fprep<<<dim3((FM * WROW + 255) / 256), 256, 0, st>>>(W, reinterpret_cast<_Float16*>(w + p.off_cP),
                                                      a.ctrl, nctrl);
  hipError_t e = hipGetLastError();
  timing_after(st, "fprep");
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int items = a.BH * (a.nsplit + a.nqb);
  const int grid = cus < items ? cus : items;
  // (the ReLU features take the three-kernel path: this kernel's ReLU form
  // spills in its key loop)
  if (p.relu) return hipErrorInvalidValue;
  timing_before(st);
  fused<false><<<dim3(grid), FNT, 0, st>>>(a);
  e = hipGetLastError();
  timing_after(st, "fused");
  return e;
}

bool fused_causal_keys_supported(int32_t d, int32_t m, int32_t dtype, int32_t relu) {
  return d == FD && m == FM && dtype == FAVOR_BF16 && !relu;
}

hipError_t fused_causal_key_states(const Plan& p, const void* K, const void* V, const float* W,
                                   float* T, float* cs, hipStream_t st, bool all_segments) {
  const int nneed = all_segments ? p.nseg : p.nseg - 1;
  if (nneed < 1) return hipSuccess;
  Args a{};
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.W32 = W;
  a.T = T;
  a.cs = cs;
  a.L = p.L;
  a.BH = p.BH;
  a.nsplit = p.nseg;
  a.seg = p.seg;
  a.knorm = p.knorm;
  const int npair = (nneed + 1) / 2;
  timing_before(st);
  ckey<<<dim3(p.BH * npair), FNT, 0, st>>>(a, npair, nneed);
  const hipError_t e = hipGetLastError();
  timing_after(st, "ckey");
  return e;
}

}  // namespace favor
