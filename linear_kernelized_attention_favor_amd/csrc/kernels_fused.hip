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
//           the eight accelerator dies (XCDs, each with its own L2) in turn,
//           and each die's work-groups take work items from their die's queue
//           (then from the other dies' queues once theirs is empty): first
//           the key items (head, 64-feature block), then the query items
//           (head, query block).  A key item computes its block's columns of
//           the state [(K')^T V | (K')^T 1] over every token of the head (the
//           four blocks of a head read the same K and V through one L2),
//           writes them as the query side's bf16 operand and arrives at the
//           head.  A query item stages W', waits for the head's four blocks,
//           stages the state and applies it to its tokens.  Items are taken
//           in queue order, so a query item only waits for key items that
//           running work-groups already hold: the wait always ends.
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
// per-feature references (set from each wave's first tile, raised lazily:
// the slow key loop), and a query tile whose denominators leave
// [2^-100, 2^100] (or whose head carries references) is redone with a
// per-row reference from its exact row maximum (the slow query tile).
// Every shift is exact: per-feature key shifts are compensated on the query
// exponent, per-row query shifts cancel in D^-1.
//
// Exchange between work-groups: the state, its references and the arrival
// counts are written with device-scope (sc1) stores, which write through to
// the device's coherence point, and read with device-scope loads; a
// work-group waits for its stores to complete (vmcnt 0) before it signals
// with a device-scope atomic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

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
constexpr int NFB = FM / 64;      // feature blocks (key items) per head
constexpr int FNCH = FM / 64;     // 64-feature chunks of the query side
constexpr int WROW = FD + 8;      // fp16 per W' row (workspace and LDS)
constexpr int KZROW = FM + 8;     // bf16 per state row (workspace and LDS)
constexpr int KZROWS = FD + 16;   // state rows: 64 value columns, z, zero rows to 80
constexpr int QTILE = 32;         // tokens per query tile (two 16-token columns)
constexpr int NXCD = 8;           // accelerator dies of the part

constexpr float kKeyBiasF = 40.0f;   // slow key loop: features start at <= 2^-40
constexpr unsigned kSpinLimit = 1u << 25;   // ~1 s of polling before giving up

// LDS of the key phase, per wave: a three-slot ring of V tiles ([32][64]
// bf16 rows of 128 bytes, the 16-byte units of row r XOR-swizzled by r & 7)
// and the tile's negated norm terms.
constexpr int VT_BYTES = FTT * FD * 2;
constexpr int KW_NB = 3 * VT_BYTES;            // offset of the norms in a wave's area
constexpr int KW_BYTES = 3 * VT_BYTES + FTT * 4;
// The waves' merge: per lane 20 accumulator quads and the references.
constexpr int MERGE_SLOT = 21 * 64 * 16;
// The finished block [65][64] fp32 and its references.
constexpr int BLK_BYTES = (FD + 1) * 64 * 4 + 64 * 4;
// The query phase: W' [256][72] fp16, the state [80][264] bf16, c [256] fp32.
constexpr int QW_BYTES = FM * WROW * 2;
constexpr int QK_BYTES = KZROWS * KZROW * 2;
constexpr int QC_BYTES = FM * 4;
constexpr int QPHASE_BYTES = QW_BYTES + QK_BYTES + QC_BYTES;
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int FUSED_LDS =
    cmax(cmax(NW * KW_BYTES, (NW / 2) * MERGE_SLOT), cmax(BLK_BYTES, QPHASE_BYTES)) + 64;
static_assert(FUSED_LDS <= 160 * 1024, "LDS of one work-group");

// Control block (u32, in the workspace): one queue head per die, a timeout
// flag, then per head the arrival count of its feature blocks; each word on
// a 128-byte line of its own (atomics on one line from many work-groups
// serialize).
struct Ctrl {
  static constexpr int LINE = 32, TIMEOUT = NXCD * LINE, HEADS = NXCD + 4;
  __device__ static int next(int x) { return x * LINE; }
  __device__ static int arrive(int bh) { return (HEADS + bh) * LINE; }
};

// Device-scope (sc1) accesses: cache policy bit 4 of the buffer and
// LDS-DMA instructions on this architecture.
constexpr int kSC1 = 16;

__device__ inline void store_sc1(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_sc1(unsigned* p, unsigned x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned load_sc1(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store16_sc1(__amdgpu_buffer_rsrc_t r, int off, uint4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, r, off, 0, kSC1);
}
// A pointer known to address global memory (the item functions receive
// generic pointers, which would otherwise compile to flat instructions).
template <class T>
__device__ inline const __attribute__((address_space(1))) T* gptr(const T* p) {
  return (const __attribute__((address_space(1))) T*)(p);
}
// This wave's outstanding memory operations have completed.
__device__ inline void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
  uint16_t* O;
  uint16_t* Kz;      // [BH][80][m+8] state, bf16, query operand order
  float* cfin;       // [BH][m] its references
  unsigned* ctrl;
  int L, BH, nqb, QB;
  float knorm;
};

// The work-group's LDS, shared by the key and query phases (file scope, so
// that every function addresses it as LDS), and the last 64 bytes as a
// broadcast area for values one thread decides.
__shared__ __align__(16) unsigned char g_smem[FUSED_LDS];
__device__ inline unsigned* bcast() { return reinterpret_cast<unsigned*>(g_smem + FUSED_LDS - 64); }

// Values every lane of a wave holds alike, moved to scalar registers: the
// item functions are called (not inlined), so their arguments arrive in
// vector registers, and buffer resources built from them would otherwise
// need a loop over lanes for every load.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
template <class T>
__device__ inline T* uni(T* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ inline Args uni(const Args& a) {
  Args u;
  u.Q = uni(a.Q); u.K = uni(a.K); u.V = uni(a.V); u.W16 = uni(a.W16); u.O = uni(a.O);
  u.Kz = uni(a.Kz); u.cfin = uni(a.cfin); u.ctrl = uni(a.ctrl);
  u.L = uni(a.L); u.BH = uni(a.BH); u.nqb = uni(a.nqb); u.QB = uni(a.QB); u.knorm = uni(a.knorm);
  return u;
}

// Sum over the four lanes {l, l^16, l^32, l^48} (one column of a 16x16 tile).
__device__ inline float colsum4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// ---------------------------------------------------------------------------
// Key pass (one wave): the head's 32-token tiles w, w + 8, ... for the 64
// features [f0, f0 + 64) (W' operands in registers).  Per tile: K straight
// from memory into the projection's operand registers (bf16 -> fp16), each
// token's -knorm |k|^2 log2(e) summed across the four lanes that hold the
// token and moved through LDS to the lanes that hold its row of the product
// (-inf past the sequence); V into the wave's LDS ring by DMA two tiles
// ahead, read back as the contraction's operand with transposing LDS reads
// (4 consecutive tokens of one column per read); S = K W'^T - n on the matrix
// cores (the norm as the C input; the slow loop subtracts the reference c_r
// there too), K~ = exp2(S) in bf16 and [V | 1]^T K~ accumulated in fp32.
// Iteration i converts and projects tile i + 1 while tile i is contracted;
// no barrier: the waves of the work-group run independently.
// ---------------------------------------------------------------------------
template <bool RELU, bool SLOW>
__device__ __forceinline__ void key_pass(const Args& a, int bh, int f0, f32x4 (&acc)[5][4],
                                         float (&cref)[4]) {
  const int lane = threadIdx.x & 63, wave = uni(static_cast<int>(threadIdx.x) >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  unsigned char* const kw = g_smem + wave * KW_BYTES;
  float* const nb = reinterpret_cast<float*>(kw + KW_NB);
  const int L = a.L;
  const int ntl = (L + FTT - 1) / FTT;                              // tiles of the head
  const int ntw = wave < ntl ? (ntl - wave + NW - 1) / NW : 0;      // this wave's tiles
  const size_t base = static_cast<size_t>(bh) * L * FD;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(a.K + base, L * FD * 2);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(a.V + base, L * FD * 2);
  auto tok0 = [&](int i) { return (wave + NW * i) * FTT; };

  f16x8 wb[4][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      wb[nt][ks] = *gptr(reinterpret_cast<const f16x8*>(a.W16 + (f0 + 16 * nt + l16) * WROW +
                                                        32 * ks + 8 * g));
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) cref[nt] = 0.f;
  if (ntw == 0) return;

  // K operand (raw bf16): token tok0(i) + 16 mt + l16, dims 32 ks + 8 g .. + 7
  // (rows past the sequence read zero).
  uint4 kraw[2][2];
  auto kload = [&](int i) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kraw[mt][ks] = buffer_load16(rk, ((tok0(i) + 16 * mt + l16) * FD + 32 * ks + 8 * g) * 2);
  };
  // V tile i into ring slot sl (4 DMA instructions; instruction j fills LDS
  // units 64 j + lane: row u / 8 holds at unit u % 8 the row's global unit
  // (u % 8) ^ (row & 7); rows past the sequence read zero).
  auto vdma = [&](int i, int sl) {
    const int tb = tok0(i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = 64 * j + lane, row = u >> 3, gu = (u & 7) ^ (row & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_ptr)(kw + sl * VT_BYTES + 1024 * j), 16,
          ((tb + row) * FD + 8 * gu) * 2, 0, 0, 0);
    }
  };
  using KOp = f16x8[2][2];
  // fp16 operands of tile i and the C input -n per product row (from LDS).
  auto prep = [&](int i, KOp& ka, f32x4 (&nq)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 x = kraw[mt][ks];
        const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
        uint4 h;
        h.x = bf16x2_to_f16x2(x.x); h.y = bf16x2_to_f16x2(x.y);
        h.z = bf16x2_to_f16x2(x.z); h.w = bf16x2_to_f16x2(x.w);
        ka[mt][ks] = __builtin_bit_cast(f16x8, h);
      }
      ss = colsum4(ss);
      const bool live = tok0(i) + 16 * mt + l16 < L;
      if (g == 0) nb[16 * mt + l16] = live ? -(a.knorm * kLog2e) * ss : -INFINITY;
    }
    wave_lds_fence();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) nq[mt] = *reinterpret_cast<const f32x4*>(&nb[16 * mt + 4 * g]);
  };
  using SArr = f32x4[2][4];
  auto proj = [&](const KOp& ka, const f32x4 (&nq)[2], SArr& S) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 c = nq[mt];
        if constexpr (SLOW) c -= cref[nt];
        S[mt][nt] = mma_f16(ka[mt][0], wb[nt][0], c);
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
  // (slow loop) some feature reached 2, or is not finite
  auto overflow = [&](const bf16x8 (&kb)[4]) {
    uint32_t o = 0;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint4 w = __builtin_bit_cast(uint4, kb[nt]);
      o |= w.x | w.y | w.z | w.w;
    }
    return __ballot((o & 0x40004000u) != 0) != 0;
  };
  // (slow loop) reference update from the tile's exact per-feature maximum:
  // set on the wave's first tile kKeyBias above it, later raised where
  // exceeded (the accumulators and the projected tile move along).
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
  // [V | 1]^T K~ for the tile in slot sl: operand row = value column 16 mv +
  // l16, positions 8 g + 0..3 / 4..7 = tokens 4 g + 0..3 / 16 + 4 g + 0..3
  // (read r: lane l16 of the 16-lane group g addresses row 16 r + 4 g + l16/4,
  // columns 16 mv + 4 (l16 % 4) .. + 3, and receives column 16 mv + l16 of
  // rows 16 r + 4 g .. + 3).
  auto contract = [&](int sl, const bf16x8 (&kb)[4]) {
    // The eight transposing reads of the tile are issued together and waited
    // for in the same statement (the compiler would otherwise wait for every
    // LDS DMA in flight before each of them; the DMA of this tile has
    // landed, see the explicit wait of the iteration).
    const uint32_t vt = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kw + sl * VT_BYTES));
    const int row = 4 * g + (l16 >> 2);
    uint32_t ad[4];
#pragma unroll
    for (int mv = 0; mv < 4; ++mv)
      ad[mv] = vt + row * 128 + (((2 * mv + ((l16 & 3) >> 1)) ^ (row & 7)) * 16) + (l16 & 1) * 8;
    uint64_t h[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(h[4]), "=&v"(h[5]),
          "=&v"(h[6]), "=&v"(h[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
#pragma unroll
    for (int mv = 0; mv < 4; ++mv) {
      const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(static_cast<uint32_t>(h[2 * mv]),
                                                              static_cast<uint32_t>(h[2 * mv] >> 32),
                                                              static_cast<uint32_t>(h[2 * mv + 1]),
                                                              static_cast<uint32_t>(h[2 * mv + 1] >> 32)));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mv][nt] = mma_bf16(va, kb[nt], acc[mv][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[4][nt] = mma_bf16(ones, kb[nt], acc[4][nt]);
  };

  // Prologue: V of tile 0, K of tile 0, V of tile 1 in flight; tile 0
  // projected (its K arrived, so V of tile 0 did) and its features formed; K
  // of tile 1 in flight.  Every load is issued even past the wave's last tile
  // (those rows read zero), so that the count of memory operations in flight
  // is the same in every iteration.
  vdma(0, 0);
  kload(0);
  vdma(1, 1);
  bf16x8 kbA[4], kbB[4];
  {
    KOp ka;
    f32x4 nq[2];
    prep(0, ka, nq);
    SArr S;
    proj(ka, nq, S);
    if constexpr (SLOW) rebase(S, true);
    features(S, kbA);
  }
  kload(1);
  // Iteration i (slot i % 3 holds V of tile i): DMA V of tile i + 2; wait
  // until V of tile i has landed (issued after it: K of tile i, V and K of
  // tile i + 1, V of tile i + 2, four operations each); convert tile i + 1
  // (its K has arrived), load K of tile i + 2, project tile i + 1, contract
  // tile i, form tile i + 1's features.
  auto step = [&](auto R, int i, const bf16x8 (&kcur)[4], bf16x8 (&knext)[4]) {
    constexpr int r = decltype(R)::value;
    __builtin_amdgcn_sched_barrier(0);
    vdma(i + 2, (r + 2) % 3);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    KOp ka;
    f32x4 nq[2];
    prep(i + 1, ka, nq);
    kload(i + 2);
    SArr S;
    proj(ka, nq, S);
    contract(r % 3, kcur);
    features(S, knext);
    if constexpr (SLOW) {
      if (__builtin_expect(overflow(knext), 0)) {
        rebase(S, false);
        features(S, knext);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int i = 0; i < ntw; i += 6) {
    step(I0{}, i, kbA, kbB);
    if (i + 1 >= ntw) break;
    step(I1{}, i + 1, kbB, kbA);
    if (i + 2 >= ntw) break;
    step(I2{}, i + 2, kbA, kbB);
    if (i + 3 >= ntw) break;
    step(I0{}, i + 3, kbB, kbA);
    if (i + 4 >= ntw) break;
    step(I1{}, i + 4, kbA, kbB);
    if (i + 5 >= ntw) break;
    step(I2{}, i + 5, kbB, kbA);
  }
  // (the DMAs issued past the wave's last tile land before the ring is reused)
  vm_drain();
}

// Merge the 8 waves' sums into wave 0 (fixed order: 4..7 into 0..3, 2..3 into
// 0..1, 1 into 0), through LDS slots of 21 quads per lane; the slow form
// rescales to the larger reference.
template <bool SLOW>
__device__ __forceinline__ void key_merge(f32x4 (&acc)[5][4], float (&cref)[4]) {
  const int lane = threadIdx.x & 63, wave = uni(static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
  for (int k = NW / 2; k >= 1; k /= 2) {
    __syncthreads();
    if (wave >= k && wave < 2 * k) {
      f32x4* slot = reinterpret_cast<f32x4*>(g_smem + (wave - k) * MERGE_SLOT) + lane;
#pragma unroll
      for (int mv = 0; mv < 5; ++mv)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) slot[(mv * 4 + nt) * 64] = acc[mv][nt];
      slot[20 * 64] = f32x4{cref[0], cref[1], cref[2], cref[3]};
    }
    __syncthreads();
    if (wave < k) {
      const f32x4* slot = reinterpret_cast<const f32x4*>(g_smem + wave * MERGE_SLOT) + lane;
      const f32x4 co = slot[20 * 64];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if constexpr (SLOW) {
          const float cn = fmaxf(cref[nt], co[nt]);
          const float x = fast_exp2(cref[nt] - cn), y = fast_exp2(co[nt] - cn);
#pragma unroll
          for (int mv = 0; mv < 5; ++mv) acc[mv][nt] = acc[mv][nt] * x + slot[(mv * 4 + nt) * 64] * y;
          cref[nt] = cn;
        } else {
#pragma unroll
          for (int mv = 0; mv < 5; ++mv) acc[mv][nt] += slot[(mv * 4 + nt) * 64];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key item (head bh, feature block fb): the fast pass and merge; if the sums
// are not finite, or some feature's ones-column sum fell below 2^-100 (its
// features underflow without a reference), the slow pass and merge.  Wave 0
// stages the block [65][64] fp32 and its references in LDS; the work-group
// writes its columns of the state as the query side's operand (row r,
// features 32 b + {4 q + i, 16 + 4 q + i} at positions 32 b + 8 q + {i, 4 + i};
// rows 65..79 zero) and of cfin with 16-byte device-scope stores, waits for
// them and arrives at its head.
// ---------------------------------------------------------------------------
template <bool RELU>
__device__ __attribute__((noinline)) void key_item(Args a_in, int bh_in, int fb_in) {
  const Args a = uni(a_in);
  const int bh = uni(bh_in), fb = uni(fb_in);
  unsigned* const bc = bcast();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6), l16 = lane & 15, g = lane >> 4;
  f32x4 acc[5][4];
  float cref[4];
  key_pass<RELU, false>(a, bh, 64 * fb, acc, cref);
  key_merge<false>(acc, cref);
  if constexpr (!RELU) {
    bool bad = false;
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) bad |= !__builtin_isfinite(acc[i][nt][v]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bad |= !(acc[4][nt][0] >= 0x1p-100f);
    }
    if (tid == 0) bc[0] = 0u;
    __syncthreads();
    if (bad) bc[0] = 1u;
    __syncthreads();
    if (bc[0]) {
      key_pass<RELU, true>(a, bh, 64 * fb, acc, cref);
      key_merge<true>(acc, cref);
    }
  }
  float* const BL = reinterpret_cast<float*>(g_smem);            // [65][64]
  float* const BLc = BL + (FD + 1) * 64;                         // [64]
  __syncthreads();   // the merge slots (shared with BL) have been read
  if (wave == 0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int f = 16 * nt + l16;
#pragma unroll
      for (int mv = 0; mv < 4; ++mv)
#pragma unroll
        for (int v = 0; v < 4; ++v) BL[(16 * mv + 4 * g + v) * 64 + f] = acc[mv][nt][v];
      if (g == 0) {
        BL[FD * 64 + f] = acc[4][nt][0];
        BLc[f] = cref[nt];
      }
    }
  }
  __syncthreads();
  {
    const __amdgpu_buffer_rsrc_t rk =
        buffer_rsrc(a.Kz + static_cast<size_t>(bh) * KZROWS * KZROW, KZROWS * KZROW * 2);
    for (int e = tid; e < KZROWS * 8; e += FNT) {
      const int row = e >> 3, b = (e >> 2) & 1, q = e & 3;
      uint4 o = make_uint4(0, 0, 0, 0);
      if (row <= FD) {
        const float4 x = *reinterpret_cast<const float4*>(BL + row * 64 + 32 * b + 4 * q);
        const float4 y = *reinterpret_cast<const float4*>(BL + row * 64 + 32 * b + 16 + 4 * q);
        o = make_uint4(pack_bf16(x.x, x.y), pack_bf16(x.z, x.w), pack_bf16(y.x, y.y),
                       pack_bf16(y.z, y.w));
      }
      store16_sc1(rk, (row * KZROW + 64 * fb + 32 * b + 8 * q) * 2, o);
    }
    if (tid < 16) {
      const __amdgpu_buffer_rsrc_t rf =
          buffer_rsrc(a.cfin + static_cast<size_t>(bh) * FM + 64 * fb, 64 * 4);
      store16_sc1(rf, 16 * tid, reinterpret_cast<const uint4*>(BLc)[tid]);
    }
  }
  vm_drain();
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_add(a.ctrl + Ctrl::arrive(bh), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Query side.  A query item is block qb of head bh, tokens [qb QB,
// min(L, (qb+1) QB)), in 32-token tiles (wave w takes tiles w, w + 8, ...).
// LDS: W' [256][72] fp16, the state [80][264] bf16 and the references c
// [256] fp32.  Per tile, for each 64-feature chunk: S^T = W' Q^T - n_q (the
// query norm |q|^2 log2(e) / 2 as the C input: a per-row shift that cancels
// in D^-1 and bounds the exponent by |w|^2 log2(e) / 2), Q~ = exp2(S^T) in
// bf16, and [KV | z]^T Q~^T accumulated in fp32; the next chunk is projected
// while the current one is applied.  O = num / den.  A tile whose
// denominators leave [2^-100, 2^100], or any tile of a head whose state
// carries references, is computed by the slow tile: the exact row maximum of
// s + c_r first, then exp2(s + c_r - M) with the shift on the vector units.
// ---------------------------------------------------------------------------
using Qraw = uint4[2][2];
using Qop = f16x8[2][2];
using QS = f32x4[4][2];
using QFeat = bf16x8[2][2];   // [kb][nt]: lane = token, 8 features (perm_of)
using QAcc = f32x4[5][2];

struct QTile {
  const _Float16* Wl;
  const uint16_t* Kzl;
  const float* cl;
  uint16_t* O;        // output rows of the head
  int q1;             // end of the block (tokens)
  int l16, g;

  // S^T (+ C) for chunk ch: rows features 64 ch + 16 mt + 4 g + v, column token.
  __device__ __forceinline__ void proj(int ch, const Qop& qop, const f32x4 (&cq)[2], QS& S) const {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 wa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        wa[mt] = *reinterpret_cast<const f16x8*>(&Wl[(64 * ch + 16 * mt + l16) * WROW + 32 * ks + 8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          S[mt][nt] = mma_f16(wa[mt], qop[nt][ks], ks == 0 ? cq[nt] : S[mt][nt]);
    }
  }
  template <bool RELU>
  __device__ __forceinline__ static void features(const QS& S, QFeat& qt) {
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
  }
  __device__ __forceinline__ void apply(int ch, const QFeat& qt, QAcc& acc) const {
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
  }
  __device__ __forceinline__ static void reset(QAcc& acc) {
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // den of token column l16 (row 64: tile 4, row 0, held by lanes g = 0).
  __device__ __forceinline__ float den_of(const QAcc& acc, int nt) const {
    return __shfl(acc[4][nt][0], l16, 64);
  }
  // O rows of the tile through a buffer resource of the block's rows [0,
  // q1): stores past the block are dropped.
  __device__ __forceinline__ void store(const QAcc& acc, int tt) const {
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(uni(O), uni(q1) * FD * 2);
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
  }
};

// Q^T operands of a 32-token tile (tokens tt + 16 nt + l16, dims 32 ks + 8 g
// .. + 7) from the head's rows through a buffer resource of the block's rows
// [0, q1): rows past the block read zeros.
__device__ __forceinline__ void q_load(__amdgpu_buffer_rsrc_t rq, int tt, int l16, int g,
                                       Qraw& raw) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      raw[nt][ks] = buffer_load16(rq, ((tt + 16 * nt + l16) * FD + 32 * ks + 8 * g) * 2);
}
template <bool RELU>
__device__ __forceinline__ void q_convert(const Qraw& r, Qop& qop, float (&nq)[2]) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 x = r[nt][ks];
      const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
      uint4 h;
      h.x = bf16x2_to_f16x2(x.x); h.y = bf16x2_to_f16x2(x.y);
      h.z = bf16x2_to_f16x2(x.z); h.w = bf16x2_to_f16x2(x.w);
      qop[nt][ks] = __builtin_bit_cast(f16x8, h);
    }
    nq[nt] = RELU ? 0.f : -0.5f * kLog2e * colsum4(ss);
  }
}

// The slow tile (rare: kept out of line, reloading its Q tile, so that the
// fast loop keeps its registers).
template <bool RELU>
__device__ __attribute__((noinline)) void query_slow_tile(QTile t, const uint16_t* Qh, int tt) {
  Qraw raw;
  q_load(buffer_rsrc(uni(Qh), uni(t.q1) * FD * 2), tt, t.l16, t.g, raw);
  Qop qop;
  float unused[2];
  q_convert<RELU>(raw, qop, unused);
  const f32x4 zq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float mx[2] = {-INFINITY, -INFINITY};
  for (int ch = 0; ch < FNCH; ++ch) {
    QS S;
    t.proj(ch, qop, zq, S);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float c = t.cl[64 * ch + 16 * mt + 4 * t.g + v];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) mx[nt] = fmaxf(mx[nt], S[mt][nt][v] + c);
      }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) mx[nt] = colmax4(mx[nt]);
  QAcc acc;
  QTile::reset(acc);
  for (int ch = 0; ch < FNCH; ++ch) {
    QS S;
    t.proj(ch, qop, zq, S);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float c = t.cl[64 * ch + 16 * mt + 4 * t.g + v];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[mt][nt][v] += c - mx[nt];
      }
    QFeat qt;
    QTile::features<RELU>(S, qt);
    t.apply(ch, qt, acc);
  }
  t.store(acc, tt);
}

template <bool RELU>
__device__ __attribute__((noinline)) void query_item(Args a_in, int bh_in, int qb_in) {
  const Args a = uni(a_in);
  const int bh = uni(bh_in), qb = uni(qb_in);
  unsigned char* const smem = g_smem;
  unsigned* const bc = bcast();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  _Float16* const Wl = reinterpret_cast<_Float16*>(smem);
  uint16_t* const Kzl = reinterpret_cast<uint16_t*>(smem + QW_BYTES);
  float* const cl = reinterpret_cast<float*>(smem + QW_BYTES + QK_BYTES);
  const int L = a.L;
  const size_t base = static_cast<size_t>(bh) * L * FD;
  const int q0 = qb * a.QB, q1 = min(L, q0 + a.QB);

  // W' (written by the previous launch) straight into LDS.
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.W16);
    uint4* dst = reinterpret_cast<uint4*>(Wl);
    constexpr int n16 = FM * WROW / 8;
    for (int j = wave; 64 * j < n16; j += FNT / 64)
      if (64 * j + lane < n16) lds_dma16(src + 64 * j + lane, dst + 64 * j);
  }
  // The wave's first tile of Q, loaded while the head's state is awaited.
  const uint16_t* const Qh = a.Q + base;
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qh, q1 * FD * 2);
  const int tstep = (FNT / 64) * QTILE;
  const int tt0 = q0 + wave * QTILE;
  const int ntile = tt0 < q1 ? (q1 - tt0 + tstep - 1) / tstep : 0;
  Qraw raw;
  q_load(rq, tt0, l16, g, raw);

  // Wait until every feature block of the head has written its columns of
  // the state.
  if (tid == 0) {
    unsigned r = 0, spins = 0;
    while ((r = load_sc1(a.ctrl + Ctrl::arrive(bh))) < static_cast<unsigned>(NFB)) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins >= kSpinLimit) {
        store_sc1(a.ctrl + Ctrl::TIMEOUT, 1u);
        break;
      }
    }
    bc[0] = r >= static_cast<unsigned>(NFB) ? 1u : 0u;
    bc[1] = 0u;
  }
  __syncthreads();
  const unsigned ready = bc[0];
  // The state and its references (written by other work-groups: sc1).
  if (ready) {
    const uint4* src = reinterpret_cast<const uint4*>(a.Kz + static_cast<size_t>(bh) * KZROWS * KZROW);
    uint4* dst = reinterpret_cast<uint4*>(Kzl);
    constexpr int n16 = KZROWS * KZROW / 8;
    for (int j = wave; 64 * j < n16; j += FNT / 64)
      if (64 * j + lane < n16)
        __builtin_amdgcn_global_load_lds(src + 64 * j + lane, dst + 64 * j, 16, 0, kSC1);
    if (wave == 0 && lane < FM / 4)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const uint4*>(a.cfin + static_cast<size_t>(bh) * FM) + lane,
          reinterpret_cast<uint4*>(cl), 16, 0, kSC1);
  }
  vm_drain();
  __syncthreads();
  if (ready && tid < FM && cl[tid] != 0.f) bc[1] = 1u;   // some key reference is not 0
  __syncthreads();
  if (ready == 0u) {
    // (the wait gave up: the output of this block is marked invalid)
    for (int i = tid; i < (q1 - q0) * FD; i += FNT)
      a.O[base + static_cast<size_t>(q0) * FD + i] = 0x7FC0u;
    return;
  }
  const bool refs = bc[1] != 0u;
  const QTile T{Wl, Kzl, cl, a.O + base, q1, l16, g};

  // Fast tiles first; the tiles that need the slow form are noted (one bit
  // per tile: at most 64 per wave by the plan) and done after the loop, so
  // that no register of the fast loop is live across the out-of-line call.
  uint64_t slow = 0;
  if (RELU || !refs) {
    Qop qcur;
    float nq[2];
    QAcc acc;
    for (int ti = 0; ti < ntile; ++ti) {
      const int tt = tt0 + ti * tstep;
      q_convert<RELU>(raw, qcur, nq);
      if (ti + 1 < ntile) q_load(rq, tt + tstep, l16, g, raw);
      const f32x4 cq[2] = {f32x4{nq[0], nq[0], nq[0], nq[0]}, f32x4{nq[1], nq[1], nq[1], nq[1]}};
      QTile::reset(acc);
      QFeat FA, FB;
      {
        QS S;
        T.proj(0, qcur, cq, S);
        QTile::features<RELU>(S, FA);
      }
      auto regular = [&](const int ch, const QFeat& Fcur, QFeat& Fnext) {
        __builtin_amdgcn_sched_barrier(0);
        QS S;
        T.proj(ch + 1, qcur, cq, S);
        T.apply(ch, Fcur, acc);
        QTile::features<RELU>(S, Fnext);
      };
      regular(0, FA, FB);
      regular(1, FB, FA);
      regular(2, FA, FB);
      __builtin_amdgcn_sched_barrier(0);
      T.apply(3, FB, acc);
      if constexpr (!RELU) {
        bool bad = false;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float den = T.den_of(acc, nt);
          bad |= (tt + 16 * nt + l16 < q1) && !(den >= 0x1p-100f && den <= 0x1p100f);
        }
        if (__ballot(bad) != 0) {
          slow |= uint64_t{1} << ti;
          continue;
        }
      }
      T.store(acc, tt);
    }
  } else {
    slow = ntile >= 64 ? ~uint64_t{0} : (uint64_t{1} << ntile) - 1;
  }
  if constexpr (!RELU) {
    while (slow) {
      const int ti = __builtin_ctzll(slow);
      slow &= slow - 1;
      query_slow_tile<RELU>(T, Qh, tt0 + ti * tstep);
    }
  }
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// fused: the persistent kernel.  Die x's queue holds, for its heads
// x, x + 8, ...: the key items (head, feature block), then the query items
// (head, query block).  A work-group serves its own die's queue first, then
// the others in turn.
// ---------------------------------------------------------------------------
template <bool RELU>
__global__ __launch_bounds__(FNT, 1) void fused(Args a) {
  unsigned* const bc = bcast();
  // (this work-group's die: hardware register XCC_ID, bits 3:0)
  const int my = static_cast<int>(__builtin_amdgcn_s_getreg(20 | (3 << 11))) % NXCD;
  for (int qi = 0; qi < NXCD; ++qi) {
    const int x = (my + qi) % NXCD;
    const int nh = x < a.BH ? (a.BH - x + NXCD - 1) / NXCD : 0;
    const int nK = nh * NFB, nItems = nK + nh * a.nqb;
    for (;;) {
      if (threadIdx.x == 0)
        bc[8] = __hip_atomic_fetch_add(a.ctrl + Ctrl::next(x), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int item = static_cast<int>(bc[8]);
      __syncthreads();
      if (item >= nItems) break;
      if (item < nK) {
        key_item<RELU>(a, x + NXCD * (item / NFB), item % NFB);
      } else {
        const int q = item - nK;
        query_item<RELU>(a, x + NXCD * (q / a.nqb), q % a.nqb);
      }
    }
  }
}

}  // namespace

bool fused_bidir_supported(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype) {
  (void)L;
  return dtype == FAVOR_BF16 && d == FD && m == FM && static_cast<int64_t>(B) * H >= 64;
}

void fused_bidir_layout(Plan* p, int cus) {
  const int BH = p->BH, L = p->L;
  // Key items: one per (head, 64-feature block) over every token.
  p->seg = L;
  p->nseg = 1;
  // Query blocks: about one query item per compute unit, a multiple of 256
  // tokens (one 32-token tile per wave), at most 64 tiles per wave (the
  // query item tracks its slow tiles in a 64-bit mask).
  const int64_t want = (static_cast<int64_t>(L) * BH + cus - 1) / cus;
  int64_t qb = (want + 255) / 256 * 256;
  qb = qb < 256 ? 256 : (qb > 64 * 256 ? 64 * 256 : qb);
  p->qblk = static_cast<int32_t>(qb);
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
  a.Kz = reinterpret_cast<uint16_t*>(w + p.off_KV);
  a.cfin = reinterpret_cast<float*>(w + p.off_cfin);
  a.ctrl = reinterpret_cast<unsigned*>(w + p.off_ctrl);
  a.L = p.L;
  a.BH = p.BH;
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
  const int items = a.BH * (NFB + a.nqb);
  const int grid = cus < items ? cus : items;
  timing_before(st);
  if (p.relu)
    fused<true><<<dim3(grid), FNT, 0, st>>>(a);
  else
    fused<false><<<dim3(grid), FNT, 0, st>>>(a);
  e = hipGetLastError();
  timing_after(st, "fused");
  return e;
}

}  // namespace favor
