// Block-scaled quantization kernels for gfx950 (MI355X).
//
// Method: Lorn blog, post "浅谈低精度浮点数".
//   section "FP8":  x^ = s * round(x / s), s = alpha / 127 (INT8); the FP8
//                   quantizer uses the E4M3 / E5M2 grid with s = alpha / FMAX.
//   section "FP4 / MXFP4 / NVFP4": MXFP4 x^ = s_mx * Q_E2M1(x / s_mx) with an
//                   E8M0 scale per 32; NVFP4 s_global = amax / (6 * 448),
//                   s_block = (block_amax / 6) / s_global cast to E4M3 per 16;
//                   INT4 q in [-7, 7], s = A / 7 (per group of 128 here).
//
// Every kernel streams x once with 16-byte non-temporal loads: one "chunk"
// is 8 consecutive elements of a row (one load for BF16, two for FP32), and
// consecutive lanes own consecutive chunks, so each load instruction of a
// wave covers a contiguous 1 KiB (BF16).  Block maxima are reduced across the
// lanes that share a block with DPP (2 lanes NVFP4, 4 lanes MXFP4, 16 lanes
// INT4); per-row maxima add one LDS step across the four waves of a
// workgroup.  Codes are produced, decoded and compared with x in registers;
// no MFMA is involved (nothing is contracted).
//
// Division x / s.  The pages define v = x / s.  The fast path computes the
// correctly rounded binary32 quotient with one Markstein correction from a
// per-unit reciprocal y = RN(1/s):
//     q0 = x*y;  r = fma(s, q0, -x);  v = fma(-r, y, q0)
// which equals RN(x/s) whenever |x| <= alpha, s >= 2^-64 and |x/s| >= 2^-20
// (checked exhaustively over every BF16 x and every scale the BF16 inputs
// can produce for INT8, FP8, INT4 and NVFP4, and on random FP32 inputs).
// Below 2^-20 every grid rounds the quotient to a signed zero, which the
// correction preserves.  Units with non-finite inputs, zero or tiny scales
// take a slow path that uses the compiler's correctly rounded division.
//
// Hardware converts.  v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest
// even on the OCP E4M3 / E5M2 grids and keep the sign of zero, but do not
// saturate; the fast path never feeds them |v| beyond the midpoint above the
// largest code (|v| <= FMAX * (1 + 2^-23)), and the slow path clamps first.
// v_cvt_scalef32_pk_fp4_f32 divides by a power-of-two scale, rounds to
// nearest even and saturates to +-6; NaN is patched to code 0 on the slow
// path.  The decode converts are exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "iq_launch.h"

namespace iqk {
namespace {

typedef float f2v __attribute__((ext_vector_type(2)));
typedef short s2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ uint32_t umax16(uint32_t m) { return (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16); }

constexpr uint32_t kNonFinite = 0x7F800000u;   // absmax bits at or above: Inf or NaN present

// ---------------------------------------------------------------------------
// Input chunks: 8 consecutive elements of one row.
// ---------------------------------------------------------------------------
template <int IN> struct Chunk;

template <> struct Chunk<D_BF16> {
    uint32_t w[4];
    __device__ __forceinline__ void load(const void* base, int64_t elem) {
        u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(static_cast<const uint16_t*>(base) + elem));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
    __device__ __forceinline__ void zero() { w[0] = w[1] = w[2] = w[3] = 0; }
    // From staged 16-byte words (word k at p[k * stride]).
    __device__ __forceinline__ void set(const u4v* p, int stride) {
        (void)stride;
        const u4v v = p[0];
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
    // BF16 -> FP32 is exact: the BF16 bits are the top half of the FP32 word.
    __device__ __forceinline__ float get(int i) const {
        return (i & 1) ? as_f(w[i >> 1] & 0xFFFF0000u) : as_f(w[i >> 1] << 16);
    }
    // Absmax on the integer image of |x| (BF16 bits |x| in [0, 0x7FFF],
    // ordered like the magnitudes): per-half maxima, combined as a tree.
    __device__ __forceinline__ static uint32_t hmax(uint32_t a, uint32_t b) {
        typedef unsigned short u2s __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u2s, a), __builtin_bit_cast(u2s, b)));
    }
    __device__ __forceinline__ uint32_t absmax_word() const {
        const uint32_t a = hmax(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu);
        const uint32_t b = hmax(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu);
        return hmax(a, b);
    }
    __device__ __forceinline__ void absmax(uint32_t& m) const { m = hmax(m, absmax_word()); }
    // FP32 bits of the maximum magnitude; kNonFinite or more means an Inf or
    // NaN is present (absmax_finite then gives the maximum over the rest).
    __device__ __forceinline__ static uint32_t absmax_bits(uint32_t m) { return umax16(m) << 16; }
    __device__ __forceinline__ static uint32_t hmin(uint32_t a, uint32_t b) {
        typedef unsigned short u2s __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u2s, a), __builtin_bit_cast(u2s, b)));
    }
    // Per-half maximum and minimum of |x| (the minimum is 0 iff an exact zero is present).
    __device__ __forceinline__ void absmaxmin_word(uint32_t& mx, uint32_t& mn) const {
        const uint32_t a0 = w[0] & 0x7FFF7FFFu, a1 = w[1] & 0x7FFF7FFFu, a2 = w[2] & 0x7FFF7FFFu, a3 = w[3] & 0x7FFF7FFFu;
        mx = hmax(hmax(a0, a1), hmax(a2, a3));
        mn = hmin(hmin(a0, a1), hmin(a2, a3));
    }
    __device__ __forceinline__ static bool has_zero(uint32_t mn) { return (mn & 0xFFFFu) == 0u || (mn >> 16) == 0u; }
    // Number of nonzero elements: bit 15 of |x| + 0x7FFF (per half) is set iff |x| != 0.
    __device__ __forceinline__ uint32_t nonzero_count() const {
        uint32_t n = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) n += __builtin_popcount(((w[k] & 0x7FFF7FFFu) + 0x7FFF7FFFu) & 0x80008000u);
        return n;
    }
    // Signed range on the bit images, per half: p collects the signed
    // maximum (the largest positive x when one is present, since positive
    // BF16 bits order like their values and negatives are negative int16),
    // n the unsigned maximum (the most negative x when one is present: the
    // sign bit makes it the largest, larger magnitudes larger still), mn the
    // minimum of |x| (0 iff an exact zero is present).
    static constexpr uint32_t kMagInit = 0x7FFF7FFFu;
    __device__ __forceinline__ void range(uint32_t& p, uint32_t& n, uint32_t& mn) const {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            p = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s2v, p), __builtin_bit_cast(s2v, w[k])));
            n = hmax(n, w[k]);
            mn = hmin(mn, w[k] & 0x7FFF7FFFu);
        }
    }
    // FP32 bits of max(0, max x) and of -min(0, min x) from range(); a value
    // of kNonFinite or more means an Inf or NaN on that side.
    __device__ __forceinline__ static void range_bits(uint32_t p, uint32_t n, uint32_t& pos, uint32_t& neg) {
        const int a = (int)(int16_t)(p & 0xFFFFu), b = (int)(int16_t)(p >> 16);
        const int m = a > b ? a : b;
        pos = m > 0 ? (uint32_t)m << 16 : 0u;
        const uint32_t u = umax16(n);
        neg = (u & 0x8000u) ? (u & 0x7FFFu) << 16 : 0u;
    }
    // Maximum over the finite elements only: t = a + 0x80 is negative as
    // int16 exactly for Inf and NaN, so a signed 16-bit max skips them.
    __device__ __forceinline__ uint32_t absmax_finite() const {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t t = (w[k] & 0x7FFF7FFFu) + 0x00800080u;
            m = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s2v, m), __builtin_bit_cast(s2v, t)));
        }
        const int lo = (int)(int16_t)(m & 0xFFFFu), hi = (int)(int16_t)(m >> 16);
        const int mx = lo > hi ? lo : hi;
        return mx >= 0x80 ? (uint32_t)(mx - 0x80) << 16 : 0u;
    }
};

template <> struct Chunk<D_F32> {
    uint32_t w[8];
    __device__ __forceinline__ void load(const void* base, int64_t elem) {
        const u4v* p = reinterpret_cast<const u4v*>(static_cast<const float*>(base) + elem);
        u4v a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = 0;
    }
    __device__ __forceinline__ void set(const u4v* p, int stride) {
        const u4v a = p[0], b = p[stride];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    __device__ __forceinline__ float get(int i) const { return as_f(w[i]); }
    __device__ __forceinline__ static uint32_t hmax(uint32_t a, uint32_t b) { return a > b ? a : b; }
    __device__ __forceinline__ uint32_t absmax_word() const {
        uint32_t a[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = hmax(w[2 * k] & 0x7FFFFFFFu, w[2 * k + 1] & 0x7FFFFFFFu);
        return hmax(hmax(a[0], a[1]), hmax(a[2], a[3]));
    }
    __device__ __forceinline__ void absmax(uint32_t& m) const { m = hmax(m, absmax_word()); }
    __device__ __forceinline__ static uint32_t absmax_bits(uint32_t m) { return m; }
    __device__ __forceinline__ static uint32_t hmin(uint32_t a, uint32_t b) { return a < b ? a : b; }
    __device__ __forceinline__ void absmaxmin_word(uint32_t& mx, uint32_t& mn) const {
        uint32_t a[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = w[k] & 0x7FFFFFFFu;
        mx = hmax(hmax(hmax(a[0], a[1]), hmax(a[2], a[3])), hmax(hmax(a[4], a[5]), hmax(a[6], a[7])));
        mn = hmin(hmin(hmin(a[0], a[1]), hmin(a[2], a[3])), hmin(hmin(a[4], a[5]), hmin(a[6], a[7])));
    }
    __device__ __forceinline__ static bool has_zero(uint32_t mn) { return mn == 0u; }
    __device__ __forceinline__ uint32_t nonzero_count() const {
        uint32_t n = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) n += (w[k] & 0x7FFFFFFFu) != 0u ? 1u : 0u;
        return n;
    }
    __device__ __forceinline__ uint32_t absmax_finite() const {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t a = w[k] & 0x7FFFFFFFu;
            m = (a < 0x7F800000u && a > m) ? a : m;
        }
        return m;
    }
    // As for BF16, on whole words.
    static constexpr uint32_t kMagInit = 0x7FFFFFFFu;
    __device__ __forceinline__ void range(uint32_t& p, uint32_t& n, uint32_t& mn) const {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            p = (int)w[k] > (int)p ? w[k] : p;
            n = w[k] > n ? w[k] : n;
            mn = hmin(mn, w[k] & 0x7FFFFFFFu);
        }
    }
    __device__ __forceinline__ static void range_bits(uint32_t p, uint32_t n, uint32_t& pos, uint32_t& neg) {
        pos = (int)p > 0 ? p : 0u;
        neg = (n & 0x80000000u) ? (n & 0x7FFFFFFFu) : 0u;
    }
};

// ---------------------------------------------------------------------------
// LDS staging.  A workgroup's staging area holds NW 16-byte words per thread,
// word k of thread t at stage[k][t].  global_load_lds_dwordx4 copies one
// word per lane from HBM into LDS without passing through VGPRs: a wave's
// instruction lands its 64 lanes at consecutive words from the wave-uniform
// base &stage[k][64 * wave].  Each lane later reads back only its own words,
// so no barrier is needed between the copy and the read.  The kernels read
// the current unit from LDS, then start the copy of their next unit into the
// same words, and compute while that copy is in flight.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
constexpr unsigned kAuxNontemporal = 2;   // cache policy bits of the copy: streaming (nt)

template <int NW, int NT = kThreads> using Stage = u4v[NW][NT];

__device__ __forceinline__ void dma_word(const void* src, u4v* wave_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)wave_base, 16, 0, kAuxNontemporal);
}

// The compiler does not track the copies' LDS writes against later LDS
// reads, so both orderings are explicit:
//   wait_staged:     the copies have landed (vmcnt(0)) before the unit is read;
//   wait_lds_reads:  the reads have completed (lgkmcnt(0)) before the next
//                    copies overwrite the same words.
__device__ __forceinline__ void wait_staged() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
}
// vmcnt(N): every copy but the N most recently issued memory operations of
// the wave has landed (the counter drains in issue order).
template <int N> __device__ __forceinline__ void wait_staged_keep() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds_reads() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
}

template <int IN> struct ChunkWords { static constexpr int n = IN == D_BF16 ? 1 : 2; };

// Start copying chunk `elem` (8 elements) of x into words [w0, w0 + n) of this thread.
template <int IN, int NW, int NT = kThreads>
__device__ __forceinline__ void stage_chunk(Stage<NW, NT>& st, int w0, const void* x, int64_t elem) {
    const int wave = threadIdx.x >> 6;
    const char* src = static_cast<const char*>(x) + elem * (IN == D_BF16 ? 2 : 4);
#pragma unroll
    for (int k = 0; k < ChunkWords<IN>::n; ++k) dma_word(src + 16 * k, &st[w0 + k][64 * wave]);
}

template <int IN, int NW, int NT = kThreads>
__device__ __forceinline__ void unstage_chunk(const Stage<NW, NT>& st, int w0, Chunk<IN>& ch) {
    ch.set(&st[w0][threadIdx.x], NT);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.  DPP within rows of 16 lanes, shuffles across rows.
// ---------------------------------------------------------------------------
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max(m, m of another lane); the DPP move starts from 0, the identity of an
// unsigned max, so the compiler folds it into the max (one instruction).
template <int CTRL> __device__ __forceinline__ uint32_t dpp_max(uint32_t m) {
    return umax(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, CTRL, 0xF, 0xF, false));
}

// Max over groups of G consecutive lanes (G = 2, 4 or 16); every lane of the
// group receives the result.
template <int G> __device__ __forceinline__ uint32_t group_max(uint32_t m) {
    m = dpp_max<kQuadSwap1>(m);
    if (G >= 4) m = dpp_max<kQuadSwap2>(m);
    if (G >= 16) {
        m = dpp_max<kRowHalfMirror>(m);
        m = dpp_max<kRowMirror>(m);
    }
    return m;
}

// Max over the wave, wave-uniform (scalar) result.
__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
    m = group_max<16>(m);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)m, 31);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
    return umax(umax(a, b), umax(c, d));
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global access of the wave (vmcnt(0)), which would stall
// on the copy of the next unit issued just before; here only the LDS
// traffic (lgkmcnt) has to be complete.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Max over the NWAVES waves of a workgroup (one LDS slot per wave beyond the
// first).  Every thread returns the result.  A slot may be written again
// only after a barrier that every thread reaches after its reads of the
// slot, i.e. the barrier of a call on another slot: the row loops alternate
// two slots between rows and give the re-reduction of a row holding Inf or
// NaN a third one.
// Max of m and OR of the per-lane flag f over the workgroup (two LDS words
// per wave beyond the first), with the same slot discipline as block_max.
template <int NWAVES>
__device__ __forceinline__ uint32_t block_max_or(uint32_t m, bool f, bool& f_out, uint32_t (&red)[NWAVES][2]) {
    m = wave_max(m);
    uint32_t fl = __ballot(f) != 0 ? 1u : 0u;
    if (NWAVES > 1) {
        if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6][0] = m; red[threadIdx.x >> 6][1] = fl; }
        asm volatile("" ::: "memory");
        lds_barrier();
        m = red[0][0]; fl = red[0][1];
#pragma unroll
        for (int k = 1; k < NWAVES; ++k) { m = umax(m, red[k][0]); fl |= red[k][1]; }
        m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m);     // uniform: keep in scalar registers
        fl = (uint32_t)__builtin_amdgcn_readfirstlane((int)fl);
    }
    f_out = fl != 0;
    return m;
}

template <int NWAVES> __device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t (&red)[NWAVES]) {
    m = wave_max(m);
    if (NWAVES == 1) return m;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    asm volatile("" ::: "memory");
    lds_barrier();
    m = red[0];
#pragma unroll
    for (int k = 1; k < NWAVES; ++k) m = umax(m, red[k]);
    return m;
}

// ---------------------------------------------------------------------------
// Error statistics.  Sums of the fast path run in FP32 over one unit of work
// (at most a few dozen terms per lane) and are folded into FP64 per lane; the
// slow path sums in FP64 directly, which also covers units whose absmax lies
// outside [2^-40, 2^60] where FP32 squares would underflow or overflow.
// Counters come from wave ballots, so they are only ever updated in
// wave-uniform control flow: every lane then holds the same, complete count.
// Lanes without data carry zeros and contribute nothing.
// ---------------------------------------------------------------------------
constexpr float kStatLo = 0x1p-40f;   // unit absmax range of the FP32 fast path
constexpr float kStatHi = 0x1p60f;

__device__ __forceinline__ bool stat_range(float a) { return a >= kStatLo && a <= kStatHi; }

struct Stats {
    double sx2 = 0, se2 = 0, sae = 0;
    float mae = 0.f;
    uint32_t nsat = 0, nzf = 0, nnf = 0;   // wave-uniform
    uint32_t lzf = 0;                      // per lane: flushed elements counted from the codes
    float fx2 = 0.f, fe2 = 0.f, fae = 0.f; // FP32 accumulators of the current unit

    __device__ __forceinline__ void fold() {
        sx2 += (double)fx2; se2 += (double)fe2; sae += (double)fae;
        fx2 = fe2 = fae = 0.f;
    }
    // One chunk of the fast path (finite inputs, unit absmax in the FP32
    // range), called in wave-uniform control flow with a wave-uniform `sat`:
    // false when no lane's unit can hold |v| > thr, which skips the
    // saturation compares (the test is |x| > thr with SAT_X, else |v| > thr).
    // Sum of squares of BF16 inputs: one v_dot2_f32_bf16 per pair of raw
    // inputs (products of BF16 values are exact in FP32).
    // With ZC the flushed count is taken here from the x^ values: zero inputs
    // always quantize to zero, so it is #(x^ == 0) - #(x == 0), the second
    // term only evaluated when some lane of the wave produced a zero.
    // Without ZC the caller counts from the codes (count_flush).
    template <int IN, bool SAT_X, bool ZC = true>
    __device__ __forceinline__ void add8_fast(const Chunk<IN>& ch, bool sat, const float (&x)[8], const float (&v)[8],
                                              const float (&h)[8], float thr) {
        float d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = x[i] - h[i];
        if (IN == D_BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                const bf2 p = __builtin_bit_cast(bf2, ch.w[k]);
                fx2 = __builtin_amdgcn_fdot2_f32_bf16(p, p, fx2, false);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) fx2 = __builtin_fmaf(x[i], x[i], fx2);
        }
        uint64_t zm = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            fe2 = __builtin_fmaf(d[i], d[i], fe2);
            fae += __builtin_fabsf(d[i]);
            mae = __builtin_fmaxf(mae, __builtin_fabsf(d[i]));
            if (ZC) {
                const uint64_t b = __ballot(h[i] == 0.f);
                zm |= b;
                nzf += __popcll(b);
            }
        }
        if (ZC && zm != 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) nzf -= __popcll(__ballot(x[i] == 0.f));
        }
        if (sat) {
            float t = thr;
            asm volatile("" : "+v"(t));   // keep the compares inside this branch
#pragma unroll
            for (int i = 0; i < 8; ++i) nsat += __popcll(__ballot(__builtin_fabsf(SAT_X ? x[i] : v[i]) > t));
        }
    }
    // Flushed elements of one chunk: nonzero inputs minus nonzero codes (a
    // nonzero code always comes from a nonzero input).
    __device__ __forceinline__ void count_flush(uint32_t nonzero_x, uint32_t nonzero_codes) { lzf += nonzero_x - nonzero_codes; }
    // General case, wave-uniform call: non-finite inputs count but stay out
    // of sums and maxima; vs is the value tested for |vs| > thr.
    __device__ __forceinline__ void add8_slow(const float (&x)[8], const float (&vs)[8], const float (&h)[8], float thr) {
        bool sat[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sat[i] = __builtin_fabsf(vs[i]) > thr;
        add8_slow_flags(x, sat, h);
    }
    // One element of the general case (wave-uniform call).
    __device__ __forceinline__ void add1_slow(float x, bool sat, float h) {
        const bool fin = __builtin_isfinite(x);
        const double d = fin ? (double)(x - h) : 0.0;
        const double xs = fin ? (double)x : 0.0;
        sx2 = __builtin_fma(xs, xs, sx2);
        se2 = __builtin_fma(d, d, se2);
        sae += __builtin_fabs(d);
        mae = __builtin_fmaxf(mae, fin ? __builtin_fabsf(x - h) : 0.f);
        nsat += __popcll(__ballot(sat));
        nzf += __popcll(__ballot(fin && x != 0.f && h == 0.f));
        nnf += __popcll(__ballot(!fin));
    }
    // The same with the saturation of each element decided by the caller.
    __device__ __forceinline__ void add8_slow_flags(const float (&x)[8], const bool (&sat)[8], const float (&h)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool fin = __builtin_isfinite(x[i]);
            const double d = fin ? (double)(x[i] - h[i]) : 0.0;
            const double xs = fin ? (double)x[i] : 0.0;
            sx2 = __builtin_fma(xs, xs, sx2);
            se2 = __builtin_fma(d, d, se2);
            sae += __builtin_fabs(d);
            mae = __builtin_fmaxf(mae, fin ? __builtin_fabsf(x[i] - h[i]) : 0.f);
            nsat += __popcll(__ballot(sat[i]));
            nzf += __popcll(__ballot(fin && x[i] != 0.f && h[i] == 0.f));
            nnf += __popcll(__ballot(!fin));
        }
    }
};

// Fast-path sums of one chunk whose x^ is h (finite inputs, unit absmax in
// the FP32 statistics range; wave-uniform call): d = x - h (exact),
// sum d^2, sum |d|, max |d|, and sum x^2 (BF16: v_dot2 on the raw pairs).
template <int IN>
__device__ __forceinline__ void sums8(Stats& st, const Chunk<IN>& ch, const float (&x)[8], const float (&h)[8]) {
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = x[i] - h[i];
    if (IN == D_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            const bf2 p = __builtin_bit_cast(bf2, ch.w[k]);
            st.fx2 = __builtin_amdgcn_fdot2_f32_bf16(p, p, st.fx2, false);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) st.fx2 = __builtin_fmaf(x[i], x[i], st.fx2);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        st.fe2 = __builtin_fmaf(d[i], d[i], st.fe2);
        st.fae += __builtin_fabsf(d[i]);
        st.mae = __builtin_fmaxf(st.mae, __builtin_fabsf(d[i]));
    }
}

// Saturated elements of a chunk, |x| > T (T >= 0, per lane), added to the
// wave-uniform count (wave-uniform call).  Compared on the integer images
// of |x| of an opaque copy of the raw words, so the compiler keeps this
// pass apart from the cast.  For BF16, |x| > T exactly when the BF16 bits
// of |x| exceed those of T truncated to BF16.
template <int IN>
__device__ __forceinline__ void count_above(Stats& st, const Chunk<IN>& ch, float T) {
    const uint32_t tb = as_u(T);
#pragma unroll
    for (int k = 0; k < (int)(sizeof(ch.w) / 4); ++k) {
        uint32_t w = ch.w[k];
        asm volatile("" : "+v"(w));
        if (IN == D_BF16) {
            st.nsat += __popcll(__ballot((w & 0x7FFFu) > (tb >> 16)));
            st.nsat += __popcll(__ballot(((w >> 16) & 0x7FFFu) > (tb >> 16)));
        } else {
            st.nsat += __popcll(__ballot((w & 0x7FFFFFFFu) > tb));
        }
    }
}

// Exact zero inputs of a valid chunk: they always give a zero code, which
// the flushed count (zero codes of nonzero inputs) must not include.
template <int IN>
__device__ __forceinline__ void uncount_zero_inputs(Stats& st, const Chunk<IN>& ch, bool valid) {
    Chunk<IN> c = ch;
#pragma unroll
    for (int k = 0; k < (int)(sizeof(c.w) / 4); ++k) asm volatile("" : "+v"(c.w[k]));
    if (valid) st.lzf -= 8u - c.nonzero_count();
}

// Whether a unit with absmax A and scale s can hold elements with |x/s| > Q:
// exactly when A > Q * s, whose sign the single rounding of fma(Q, s, -A)
// preserves.
__device__ __forceinline__ bool can_saturate(float A, float s, float Q) { return __builtin_fmaf(Q, s, -A) < 0.f; }


// ---------------------------------------------------------------------------
// Statistics across workgroups.  Every workgroup of a launch reduces its own
// statistics to one partial, publishes it and counts its arrival; the last
// workgroup to arrive folds all partials, in a fixed order, into the output.
//   Publishing uses device-scope atomic exchanges, whose results the
//   workgroup waits for: an exchange has been performed at device scope
//   when its old value returns, so every partial is in place before its
//   arrival is counted.  Arrivals are device-scope atomic adds on counters
//   of 64 workgroups each, then on one launch-wide counter (a single
//   counter taking every workgroup's add serializes them: about 7 ns each,
//   15 us on a 2048-workgroup launch whose workgroups all end together).
//   The folding workgroup reads the partials with device-scope atomic
//   loads after its own arrival returned, i.e. after every other one.
//   No cache writeback of the whole L2 is needed, which a release fence per
//   workgroup would cost.
// ---------------------------------------------------------------------------
struct StatsOut {   // mirrors iq_stats
    uint64_t n, n_zero_flush, n_saturated, n_nonfinite;
    double sum_x2, sum_err2, sum_abs_err;
    float max_abs_err;
    uint32_t reserved;
};

struct StatsSink {
    Partial* partials;   // one slot per workgroup
    uint32_t* ticket;    // arrival counters (kTicketBytes): zero at the start and at the end
    StatsOut* out;       // may be null: the partials of an x^ call without statistics
    uint64_t nelem;
};

// Sum over the 64 lanes with a fixed butterfly (the same order on every run).
template <typename T> __device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Arrival of one workgroup (one thread), after its partial has been
// performed at device scope: true for the last workgroup of the launch.
// Counters: [0] the launch, [kTicketStride * (1 + g)] group g.  Device-scope
// atomics are performed at one point in a single order, so the last arrival
// sees every partial published before any arrival it follows.
__device__ bool arrive_last(uint32_t* tickets) {
    const uint32_t n = gridDim.x, g = blockIdx.x / kTicketGroup;
    const uint32_t left = n - g * kTicketGroup, gsize = left < (uint32_t)kTicketGroup ? left : (uint32_t)kTicketGroup;
    uint32_t* gc = tickets + kTicketStride * (1 + g);
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gsize - 1) return false;
    __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ngroups = (n + kTicketGroup - 1) / kTicketGroup;
    if (__hip_atomic_fetch_add(tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ngroups - 1) return false;
    __hip_atomic_store(tickets, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Fold the n published partials (all NT threads of the last workgroup):
// thread t folds partials t, t + NT, ... in that order, then lanes and
// waves combine in a fixed pattern.  Deterministic for a given grid.
template <int NT>
__device__ void fold_partials(const StatsSink& sink, int n) {
    constexpr int NW = NT / 64;
    __shared__ double s_d[NW][3];
    __shared__ float s_m[NW];
    __shared__ uint64_t s_c[NW][3];
    const int t = threadIdx.x;
    double a = 0.0, b = 0.0, c = 0.0;
    float m = 0.f;
    uint64_t c0 = 0, c1 = 0, c2 = 0;
    // loads go out four partials at a time, all issued before the first sum
    constexpr int PER = kMaxGrid / NT, B = PER < 4 ? PER : 4;
#pragma unroll
    for (int k0 = 0; k0 < PER; k0 += B) {
        if (k0 * NT >= n) break;   // uniform: the batches past the grid hold no partials
        uint64_t pw[B][5];
#pragma unroll
        for (int k = 0; k < B; ++k) {
            const int i = t + (k0 + k) * NT;
            const uint64_t* q = reinterpret_cast<const uint64_t*>(sink.partials + (i < n ? i : 0));
#pragma unroll
            for (int f = 0; f < 5; ++f)
                pw[k][f] = __hip_atomic_load(q + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int k = 0; k < B; ++k) {
            if (t + (k0 + k) * NT >= n) continue;
            a += __builtin_bit_cast(double, pw[k][0]);
            b += __builtin_bit_cast(double, pw[k][1]);
            c += __builtin_bit_cast(double, pw[k][2]);
            m = __builtin_fmaxf(m, as_f((uint32_t)pw[k][3]));
            c0 += (uint32_t)(pw[k][3] >> 32);
            c1 += (uint32_t)pw[k][4];
            c2 += (uint32_t)(pw[k][4] >> 32);
        }
    }
    a = wave_sum(a); b = wave_sum(b); c = wave_sum(c);
    c0 = wave_sum(c0); c1 = wave_sum(c1); c2 = wave_sum(c2);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
    const int w = t >> 6;
    if ((t & 63) == 0) {
        s_d[w][0] = a; s_d[w][1] = b; s_d[w][2] = c; s_m[w] = m;
        s_c[w][0] = c0; s_c[w][1] = c1; s_c[w][2] = c2;
    }
    __syncthreads();
    if (t == 0) {
        StatsOut o;
        o.n = sink.nelem;
        o.sum_x2 = s_d[0][0]; o.sum_err2 = s_d[0][1]; o.sum_abs_err = s_d[0][2]; o.max_abs_err = s_m[0];
        o.n_saturated = s_c[0][0]; o.n_zero_flush = s_c[0][1]; o.n_nonfinite = s_c[0][2];
#pragma unroll
        for (int k = 1; k < NW; ++k) {   // waves in order
            o.sum_x2 += s_d[k][0]; o.sum_err2 += s_d[k][1]; o.sum_abs_err += s_d[k][2];
            o.max_abs_err = __builtin_fmaxf(o.max_abs_err, s_m[k]);
            o.n_saturated += s_c[k][0]; o.n_zero_flush += s_c[k][1]; o.n_nonfinite += s_c[k][2];
        }
        o.reserved = 0;
        if (sink.out) *sink.out = o;
    }
}

// Reduce the workgroup's statistics (NWAVES waves) to its partial, publish
// it, and fold all partials if this workgroup finishes last.
template <int NWAVES>
__device__ void write_partial(Stats& st, const StatsSink& sink) {
    __shared__ double s_d[NWAVES][3];
    __shared__ float s_m[NWAVES];
    __shared__ uint32_t s_c[NWAVES][3];
    __shared__ uint32_t s_last;
    st.fold();
    double a = st.sx2, b = st.se2, c = st.sae;
    float m = st.mae;
    // The ballot counters were only updated in wave-uniform control flow:
    // every lane holds the wave's count; lzf is per lane.
    uint32_t lz = st.lzf;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        a += __shfl_xor(a, o); b += __shfl_xor(b, o); c += __shfl_xor(c, o);
        m = __builtin_fmaxf(m, __shfl_xor(m, o));
        lz += (uint32_t)__shfl_xor((int)lz, o);
    }
    const uint32_t n0 = st.nsat, n1 = st.nzf + lz, n2 = st.nnf;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (NWAVES > 1 && lane == 0) {
        s_d[wave][0] = a; s_d[wave][1] = b; s_d[wave][2] = c; s_m[wave] = m;
        s_c[wave][0] = n0; s_c[wave][1] = n1; s_c[wave][2] = n2;
    }
    if (NWAVES > 1) __syncthreads();
    if (threadIdx.x == 0) {
        Partial p;
        if (NWAVES == 1) {
            p.sum_x2 = a; p.sum_err2 = b; p.sum_abs_err = c; p.max_abs_err = m;
            p.n_saturated = n0; p.n_zero_flush = n1; p.n_nonfinite = n2;
        } else {
            p.sum_x2 = s_d[0][0]; p.sum_err2 = s_d[0][1]; p.sum_abs_err = s_d[0][2]; p.max_abs_err = s_m[0];
            p.n_saturated = s_c[0][0]; p.n_zero_flush = s_c[0][1]; p.n_nonfinite = s_c[0][2];
#pragma unroll
            for (int k = 1; k < NWAVES; ++k) {
                p.sum_x2 += s_d[k][0]; p.sum_err2 += s_d[k][1]; p.sum_abs_err += s_d[k][2];
                p.max_abs_err = __builtin_fmaxf(p.max_abs_err, s_m[k]);
                p.n_saturated += s_c[k][0]; p.n_zero_flush += s_c[k][1]; p.n_nonfinite += s_c[k][2];
            }
        }
        uint64_t* q = reinterpret_cast<uint64_t*>(sink.partials + blockIdx.x);
        const uint64_t r0 = __hip_atomic_exchange(q + 0, __builtin_bit_cast(uint64_t, p.sum_x2), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t r1 = __hip_atomic_exchange(q + 1, __builtin_bit_cast(uint64_t, p.sum_err2), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t r2 = __hip_atomic_exchange(q + 2, __builtin_bit_cast(uint64_t, p.sum_abs_err), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t r3 = __hip_atomic_exchange(q + 3, (uint64_t)as_u(p.max_abs_err) | ((uint64_t)p.n_saturated << 32),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t r4 = __hip_atomic_exchange(q + 4, (uint64_t)p.n_zero_flush | ((uint64_t)p.n_nonfinite << 32),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The old values are consumed here, so the exchanges have returned
        // (been performed) before the ticket below is taken.
        asm volatile("" ::"v"(r0), "v"(r1), "v"(r2), "v"(r3), "v"(r4) : "memory");
        s_last = arrive_last(sink.ticket) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last != 0) fold_partials<NWAVES * 64>(sink, (int)gridDim.x);
}

// ---------------------------------------------------------------------------
// Grids and their constants.
// ---------------------------------------------------------------------------
template <int FMT> struct Fmt;
// qmid: the midpoint between qmax and the next binary32 above it (qmax's
// significand is even, so the midpoint itself rounds down to qmax).
template <> struct Fmt<F_INT8> {
    static constexpr float qmax = 127.f; static constexpr int iq = 127;
    static constexpr double qmid = 127.0 + 0x1p-18;
};
template <> struct Fmt<F_E4M3> {
    static constexpr float qmax = 448.f; static constexpr int iq = 448;
    static constexpr double qmid = 448.0 + 0x1p-16;
};
template <> struct Fmt<F_E5M2> {
    static constexpr float qmax = 57344.f; static constexpr int iq = 57344;
    static constexpr double qmid = 57344.0 + 0x1p-9;
};
template <> struct Fmt<F_MXFP4> { static constexpr float qmax = 6.f; };
template <> struct Fmt<F_NVFP4> {
    static constexpr float qmax = 6.f;
    static constexpr double qmid = 6.0 + 0x1p-22;
};
template <> struct Fmt<F_INT4> {
    static constexpr float qmax = 7.f;
    static constexpr double qmid = 7.0 + 0x1p-22;
};
template <> struct Fmt<F_INT4ZP> { static constexpr float qmax = 15.f; };   // codes 0..15

// Saturation in the x domain: for s > 0 and the correctly rounded v = x / s,
// |v| > Q exactly when x / s > qmid (the midpoint above Q rounds down to Q),
// i.e. when |x| > T = RD(qmid * s).  The FP64 product is exact (25 + 24
// significant bits).  Checked on the CPU for every grid against the
// division, with x next to T and to Q * s over scales 2^-60 .. 2^60.
__device__ __forceinline__ float rd_to_float(double p) {   // p >= 0
    float f = (float)p;
    if ((double)f > p) f = as_f(as_u(f) - 1u);
    return f;
}
template <int FMT> __device__ __forceinline__ float sat_threshold(float s) {
    return rd_to_float(Fmt<FMT>::qmid * (double)s);
}

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds |v| < 2^22 to an integer (RNE)
constexpr float kTinyScale = 0x1p-64f;  // smaller scales take the slow path

__device__ __forceinline__ float markstein(float x, float s, float y) {
    float q0 = x * y;
    float r = __builtin_fmaf(s, q0, -x);
    return __builtin_fmaf(-r, y, q0);
}

// a / Q for a constant Q by the same correction with the compile-time
// reciprocal RN(1/Q).  Checked against the correctly rounded quotient for
// every finite binary32 a: equal for Q = 7, 15 and 127 everywhere, and for
// Q = 6, 448, 2688 and 57344 whenever the quotient is a normal number (the
// only differences have subnormal quotients); callers take the division
// for quotients below kMarksteinMin.
constexpr float kMarksteinMin = 0x1p-100f;
template <int QI> __device__ __forceinline__ float div_const(float a) {
    constexpr float Q = (float)QI, r = 1.0f / (float)QI;
    const float q0 = a * r;
    const float e = __builtin_fmaf(-Q, q0, a);
    return __builtin_fmaf(e, r, q0);
}

// Nonzero codes among the 4 bytes of w (INT8 / FP8: a code is zero iff its
// low 7 bits are, -128 is never produced): bit 7 of (c & 0x7F) + 0x7F.
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
    return __builtin_popcount(((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u);
}
// Nonzero codes among the 8 nibbles of w (E2M1 and INT4: a code is zero iff
// its low 3 bits are; INT4 never produces -8).
__device__ __forceinline__ uint32_t nonzero_nibbles(uint32_t w) {
    return __builtin_popcount(((w & 0x77777777u) + 0x77777777u) & 0x88888888u);
}
// Nibbles of w with any of their 4 bits set.
__device__ __forceinline__ uint32_t nonzero_nibbles_full(uint32_t w) {
    return __builtin_popcount((((w & 0x77777777u) + 0x77777777u) | w) & 0x88888888u);
}

// FP8 pack / unpack (4 codes per 32-bit word, element 0 in the low byte).
template <int FMT> __device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
    uint32_t w;
    if (FMT == F_E4M3) {
        w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
    } else {
        w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, (int)w, true);
    }
    return w;
}
template <int FMT, bool HI> __device__ __forceinline__ f2v fp8_unpack2(uint32_t w) {
    f2v r;
    if (FMT == F_E4M3) {
        auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
        r.x = d[0]; r.y = d[1];
    } else {
        auto d = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
        r.x = d[0]; r.y = d[1];
    }
    return r;
}
// Exact value of one E4M3 code (low byte of c).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
    return d[0];
}

// ---------------------------------------------------------------------------
// x^ output of one chunk (FP32 or BF16 by round to nearest even).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_xhat(void* xhat, int dtype, int64_t elem, const float (&h)[8]) {
    if (dtype == D_F32) {
        u4v* p = reinterpret_cast<u4v*>(static_cast<float*>(xhat) + elem);
        u4v a = {as_u(h[0]), as_u(h[1]), as_u(h[2]), as_u(h[3])};
        u4v b = {as_u(h[4]), as_u(h[5]), as_u(h[6]), as_u(h[7])};
        __builtin_nontemporal_store(a, p);
        __builtin_nontemporal_store(b, p + 1);
    } else {
        u4v o;
        uint32_t r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t w;
            asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(w) : "v"(h[2 * k]), "v"(h[2 * k + 1]));
            r[k] = w;
        }
        o.x = r[0]; o.y = r[1]; o.z = r[2]; o.w = r[3];
        __builtin_nontemporal_store(o, reinterpret_cast<u4v*>(static_cast<uint16_t*>(xhat) + elem));
    }
}

// ---------------------------------------------------------------------------
// INT8 / FP8 with a scale shared by the whole chunk (per row or per tensor).
// `fast` and `sat` are wave-uniform: fast means a finite unit with absmax in
// [2^-40, 2^60] (Markstein quotient, FP32 statistics), sat that some lane's
// unit can saturate.  Every lane computes (lanes without data hold zeros);
// only lanes with `store` write their 8 code bytes at codes8.  h receives x^.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ void cast_uniform_fast(const float (&x)[8], float s, float y, float (&v)[8], float (&h)[8],
                                                  uint32_t& w0, uint32_t& w1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = markstein(x[i], s, y);
    if (FMT == F_INT8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t[i] = v[i] + kMagic;        // |v| <= 127 * (1 + 2^-23): the sum is the RNE integer
            h[i] = s * (t[i] - kMagic);  // (t - kMagic) is +0 for a zero code
        }
        const uint32_t p0 = __builtin_amdgcn_perm(as_u(t[1]), as_u(t[0]), 0x0c0c0400u);
        const uint32_t p1 = __builtin_amdgcn_perm(as_u(t[3]), as_u(t[2]), 0x0c0c0400u);
        const uint32_t p2 = __builtin_amdgcn_perm(as_u(t[5]), as_u(t[4]), 0x0c0c0400u);
        const uint32_t p3 = __builtin_amdgcn_perm(as_u(t[7]), as_u(t[6]), 0x0c0c0400u);
        w0 = p0 | (p1 << 16);
        w1 = p2 | (p3 << 16);
    } else {
        w0 = fp8_pack4<FMT>(v[0], v[1], v[2], v[3]);
        w1 = fp8_pack4<FMT>(v[4], v[5], v[6], v[7]);
        const f2v d0 = fp8_unpack2<FMT, false>(w0), d1 = fp8_unpack2<FMT, true>(w0);
        const f2v d2 = fp8_unpack2<FMT, false>(w1), d3 = fp8_unpack2<FMT, true>(w1);
        h[0] = s * d0.x; h[1] = s * d0.y; h[2] = s * d1.x; h[3] = s * d1.y;
        h[4] = s * d2.x; h[5] = s * d2.y; h[6] = s * d3.x; h[7] = s * d3.y;
    }
}

// Slow path: correctly rounded division, explicit clamps and NaN codes.
template <int FMT>
__device__ __forceinline__ void cast_uniform_slow(const float (&x)[8], float s, float (&v)[8], float (&h)[8],
                                               uint32_t& w0, uint32_t& w1) {
    constexpr float Q = Fmt<FMT>::qmax;
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (s == 0.f) ? 0.f : x[i] / s;
    if (FMT == F_INT8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v[i]), -127.f), 127.f);
            const int qi = __builtin_isnan(v[i]) ? 0 : (int)q;   // via int: a zero code is +0
            c[i] = (uint32_t)qi & 0xFFu;
            h[i] = s * (float)qi;
        }
    } else {
        float cl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cl[i] = __builtin_fminf(__builtin_fmaxf(v[i], -Q), Q);
        const uint32_t a = fp8_pack4<FMT>(cl[0], cl[1], cl[2], cl[3]);
        const uint32_t b = fp8_pack4<FMT>(cl[4], cl[5], cl[6], cl[7]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t byte = ((i < 4 ? a : b) >> (8 * (i & 3))) & 0xFFu;
            if (__builtin_isnan(v[i])) byte = 0x7Fu;
            if (s == 0.f) byte = 0u;
            c[i] = byte;
        }
        const uint32_t a2 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        const uint32_t b2 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        const f2v d0 = fp8_unpack2<FMT, false>(a2), d1 = fp8_unpack2<FMT, true>(a2);
        const f2v d2 = fp8_unpack2<FMT, false>(b2), d3 = fp8_unpack2<FMT, true>(b2);
        h[0] = s * d0.x; h[1] = s * d0.y; h[2] = s * d1.x; h[3] = s * d1.y;
        h[4] = s * d2.x; h[5] = s * d2.y; h[6] = s * d3.x; h[7] = s * d3.y;
    }
    w0 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w1 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
}

// Fast path of a unit (finite, absmax in the fast range), wave-uniform
// `sat` and `zeros`: `zeros` means the unit may hold exact zeros; without
// it every lane with `store` holds 8 nonzero inputs and lanes without data
// hold zeros.
// T = sat_threshold(s): the saturation count compares |x| > T, so the
// quotients are dead once converted.  SAT and ZEROS fixed at compile time
// keep the unrolled chunks free of branches (runtime flags inside the
// chunk loop cost about 30 VGPRs).
template <int IN, int FMT, bool STATS, bool SAT, bool ZEROS>
__device__ __forceinline__ void quant_chunk_fast_t(const Chunk<IN>& ch, float s, float y, float T, bool store,
                                                   uint8_t* codes8, float (&h)[8], Stats& st) {
    float x[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ch.get(i);
    uint32_t w0, w1;
    cast_uniform_fast<FMT>(x, s, y, v, h, w0, w1);
    if (STATS) {
        st.add8_fast<IN, true, false>(ch, SAT, x, v, h, T);
        st.count_flush(ZEROS ? ch.nonzero_count() : (store ? 8u : 0u), nonzero_bytes(w0) + nonzero_bytes(w1));
    }
    if (store) {
        const u2v o = {w0, w1};
        __builtin_nontemporal_store(o, reinterpret_cast<u2v*>(codes8));
    }
}

template <int IN, int FMT, bool STATS>
__device__ __forceinline__ void quant_chunk_fast(const Chunk<IN>& ch, float s, float y, bool sat, float T, bool zeros,
                                                 bool store, uint8_t* codes8, float (&h)[8], Stats& st) {
    if (sat) {
        if (zeros) quant_chunk_fast_t<IN, FMT, STATS, true, true>(ch, s, y, T, store, codes8, h, st);
        else quant_chunk_fast_t<IN, FMT, STATS, true, false>(ch, s, y, T, store, codes8, h, st);
    } else {
        if (zeros) quant_chunk_fast_t<IN, FMT, STATS, false, true>(ch, s, y, T, store, codes8, h, st);
        else quant_chunk_fast_t<IN, FMT, STATS, false, false>(ch, s, y, T, store, codes8, h, st);
    }
}

// General path: correctly rounded division, clamps, FP64 statistics.
template <int IN, int FMT, bool STATS>
__device__ __forceinline__ void quant_chunk_slow(const Chunk<IN>& ch, float s, bool store, uint8_t* codes8,
                                                 float (&h)[8], Stats& st) {
    constexpr float Q = Fmt<FMT>::qmax;
    float x[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ch.get(i);
    uint32_t w0, w1;
    cast_uniform_slow<FMT>(x, s, v, h, w0, w1);
    if (STATS) st.add8_slow(x, v, h, Q);
    if (store) {
        const u2v o = {w0, w1};
        __builtin_nontemporal_store(o, reinterpret_cast<u2v*>(codes8));
    }
}

template <int IN, int FMT, bool STATS>
__device__ __forceinline__ void quant_chunk_uniform(const Chunk<IN>& ch, float s, float y, bool fast, bool sat, float T,
                                                    bool zeros, bool store, uint8_t* codes8, float (&h)[8], Stats& st) {
    if (fast) quant_chunk_fast<IN, FMT, STATS>(ch, s, y, sat, T, zeros, store, codes8, h, st);
    else quant_chunk_slow<IN, FMT, STATS>(ch, s, store, codes8, h, st);
}

// ---------------------------------------------------------------------------
// Per-row INT8 / FP8.  A workgroup of NT threads (one wave for rows of up to
// 1024 chunks, four waves for longer ones) owns one row at a time and keeps
// it in registers between the absmax and the cast, CPT chunks per thread.
// ---------------------------------------------------------------------------
struct RowArgs {
    const void* x;
    int64_t ld;
    int32_t rows, cpr;   // chunks per row
    uint8_t* codes;
    float* scales;
    void* xhat;
    int xhat_dtype;
    StatsSink sink;
    // per-tensor scale over rows of the tensor (TENSOR): the absmax
    // pre-pass's words and where the tensor's scale goes
    const uint64_t* amax_words;
    int32_t amax_nwords;
    float* scale_out;
};

template <int IN, int CPT, int NT>
using RowStage = Stage<CPT * ChunkWords<IN>::n, NT>;

// FULL: the row has exactly CPT * NT chunks (every lane holds data).  The
// row address is scalar; each lane adds its own 32-bit byte offset, and
// `wave` (uniform) selects the wave's LDS words.
template <int IN, int CPT, int NT, bool FULL>
__device__ __forceinline__ void stage_row(RowStage<IN, CPT, NT>& st, const RowArgs& a, int32_t row, int wave) {
    constexpr int W = ChunkWords<IN>::n;
    const char* rp = static_cast<const char*>(a.x) + (int64_t)row * a.ld * (IN == D_BF16 ? 2 : 4);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t c = threadIdx.x + j * NT;
        if (FULL || (int)c < a.cpr) {
#pragma unroll
            for (int k = 0; k < W; ++k) dma_word(rp + (c * 16u * W + 16u * k), &st[j * W + k][64 * wave]);
        }
    }
}

template <int IN, int CPT, int NT, bool FULL>
__device__ __forceinline__ void unstage_row(const RowStage<IN, CPT, NT>& st, const RowArgs& a, Chunk<IN> (&ch)[CPT]) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        if (FULL || (int)threadIdx.x + j * NT < a.cpr) unstage_chunk<IN, CPT * ChunkWords<IN>::n, NT>(st, j * ChunkWords<IN>::n, ch[j]);
        else ch[j].zero();
    }
}

// Rows in flight per workgroup of the per-row kernels: two LDS buffers for
// FULL BF16 rows of 2048 chunks (16384 columns, 8 waves of 4 chunks per
// lane), one elsewhere.
template <int IN, int CPT, int NT, bool FULL>
constexpr int kRowDepth = FULL && IN == D_BF16 && CPT * NT >= 2048 ? 2 : 1;

// Row scale and flags, uniform over the workgroup (sat: over the wave).
struct RowScale {
    float s, y, T;   // T: saturation threshold in the x domain
    bool fast, sat, zeros;
};

template <int IN, int FMT, int CPT, int NT>
__device__ __forceinline__ RowScale row_scale(const Chunk<IN> (&ch)[CPT], uint32_t (&red)[3][NT / 64][2],
                                              int parity) {
    constexpr float Q = Fmt<FMT>::qmax;
    uint32_t wm[CPT], wn[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) ch[j].absmaxmin_word(wm[j], wn[j]);
#pragma unroll
    for (int step = 1; step < CPT; step *= 2)
#pragma unroll
        for (int j = 0; j + step < CPT; j += 2 * step) {
            wm[j] = Chunk<IN>::hmax(wm[j], wm[j + step]);
            wn[j] = Chunk<IN>::hmin(wn[j], wn[j + step]);
        }
    const uint32_t lane_bits = Chunk<IN>::absmax_bits(wm[0]);
    bool zeros;
    uint32_t bits = block_max_or<NT / 64>(lane_bits, Chunk<IN>::has_zero(wn[0]), zeros, red[parity]);
    const bool nonfinite = bits >= kNonFinite;
    if (nonfinite) {   // the row holds Inf or NaN: absmax over its finite elements
        uint32_t f = 0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) f = umax(f, ch[j].absmax_finite());
        bool unused;
        bits = block_max_or<NT / 64>(f, false, unused, red[2]);
    }
    const float alpha = as_f(bits);
    RowScale r;
    r.zeros = zeros;
    // fast: finite row with alpha in [2^-40, 2^60] (so s >= 2^-64)
    r.fast = !nonfinite && stat_range(alpha);
    // alpha / Q: the constant-divisor correction is exact for normal quotients
    r.s = stat_range(alpha) ? div_const<Fmt<FMT>::iq>(alpha) : alpha / Q;
    r.y = r.fast ? 1.0f / r.s : 0.f;
    r.T = sat_threshold<FMT>(r.s);
    // only waves holding a saturating element count per element
    r.sat = !r.fast || __ballot(as_f(lane_bits) > r.T) != 0;
    return r;
}

// One element of the general path: correctly rounded division, clamps,
// NaN codes (INT8: 0; FP8: 0x7F), a zero scale giving +0 codes.
template <int FMT>
__device__ __forceinline__ uint32_t cast1_slow(float x, float s, float& v, float& h) {
    constexpr float Q = Fmt<FMT>::qmax;
    v = (s == 0.f) ? 0.f : x / s;
    if (FMT == F_INT8) {
        const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v), -127.f), 127.f);
        const int qi = __builtin_isnan(v) ? 0 : (int)q;
        h = s * (float)qi;
        return (uint32_t)qi & 0xFFu;
    } else {
        const float cl = __builtin_fminf(__builtin_fmaxf(v, -Q), Q);
        uint32_t c = fp8_pack4<FMT>(cl, 0.f, 0.f, 0.f) & 0xFFu;
        if (__builtin_isnan(v)) c = 0x7Fu;
        if (s == 0.f) c = 0u;
        h = s * fp8_unpack2<FMT, false>(c).x;
        return c;
    }
}

template <int IN> __device__ __forceinline__ float load_elem(const void* x, int64_t i) {
    if (IN == D_BF16) return as_f((uint32_t)static_cast<const uint16_t*>(x)[i] << 16);
    return static_cast<const float*>(x)[i];
}

__device__ __forceinline__ void store_xhat1(void* xhat, int dtype, int64_t i, float h) {
    if (dtype == D_F32) {
        static_cast<float*>(xhat)[i] = h;
    } else {
        uint32_t w;
        asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(w) : "v"(h), "v"(h));
        static_cast<uint16_t*>(xhat)[i] = (uint16_t)w;
    }
}

// Rows that are not finite or whose absmax leaves [2^-40, 2^60]: element by
// element, re-read from x, in rolled loops, so this rare case needs few
// registers and does not lower the kernel's occupancy.  The loops are
// uniform; lanes past the row end work on zeros and store nothing.
template <int IN, int FMT, int CPT, int NT, bool FULL, bool XHAT, bool STATS>
__device__ __forceinline__ void quant_row_slow(const RowArgs& a, int32_t row, float s, uint8_t* crow, Stats& st) {
    constexpr float Q = Fmt<FMT>::qmax;
    const int64_t base = (int64_t)row * a.ld;
    const int64_t cols = (int64_t)a.cpr * kChunk;
#pragma unroll 1
    for (int j = 0; j < CPT; ++j) {
        const uint32_t c = threadIdx.x + j * NT;
        const bool valid = FULL || (int)c < a.cpr;
        uint32_t w0 = 0, w1 = 0;
#pragma unroll 1
        for (int i = 0; i < 8; ++i) {
            const float x = valid ? load_elem<IN>(a.x, base + (int64_t)c * kChunk + i) : 0.f;
            float v, h;
            const uint32_t code = cast1_slow<FMT>(x, s, v, h);
            if (i < 4) w0 |= code << (8 * i);
            else w1 |= code << (8 * (i - 4));
            if (STATS) st.add1_slow(x, __builtin_fabsf(v) > Q, h);
            if (XHAT && valid) store_xhat1(a.xhat, a.xhat_dtype, (int64_t)row * cols + (int64_t)c * kChunk + i, h);
        }
        if (valid) {
            const u2v o = {w0, w1};
            __builtin_nontemporal_store(o, reinterpret_cast<u2v*>(crow + c * 8u));
        }
    }
}

// Fast path of a staged row.  Saturated elements and exact zeros are
// counted first, in the rare waves and rows that hold them, so that the
// cast below is one branch-free body (flags inside the unrolled chunk loop
// cost about 30 VGPRs).  Within the fast range only elements equal to the
// row's absmax can exceed T (T > the float below alpha), so `r.sat` is set
// in the waves holding the maximum when it saturates.  The cast counts zero
// codes as flushed; zero inputs, which always give a zero code, are
// subtracted here.
template <int IN, int FMT, int CPT, int NT, bool FULL, bool XHAT, bool STATS>
__device__ __forceinline__ void quant_row_fast(const Chunk<IN> (&ch)[CPT], const RowArgs& a, int32_t row,
                                               const RowScale& r, uint8_t* crow, Stats& st) {
    const int64_t cols = (int64_t)a.cpr * kChunk;
    if (STATS && r.sat) {
        // |x| > T on the integer images of |x| (opaque copies, so that none
        // of this is shared with, and hoisted for, the cast below)
        const uint32_t tb = as_u(r.T);
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
#pragma unroll
            for (int k = 0; k < (int)(sizeof(ch[j].w) / 4); ++k) {
                uint32_t w = ch[j].w[k];
                asm volatile("" : "+v"(w));
                if (IN == D_BF16) {
                    st.nsat += __popcll(__ballot((w & 0x7FFFu) > (tb >> 16)));
                    st.nsat += __popcll(__ballot(((w >> 16) & 0x7FFFu) > (tb >> 16)));
                } else {
                    st.nsat += __popcll(__ballot((w & 0x7FFFFFFFu) > tb));
                }
            }
        }
    }
    if (STATS && r.zeros) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            Chunk<IN> cj = ch[j];   // opaque copy, as above
#pragma unroll
            for (int k = 0; k < (int)(sizeof(cj.w) / 4); ++k) asm volatile("" : "+v"(cj.w[k]));
            if (FULL || (int)(threadIdx.x + j * NT) < a.cpr) st.lzf -= 8u - cj.nonzero_count();
        }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t c = threadIdx.x + j * NT;
        const bool valid = FULL || (int)c < a.cpr;
        float h[8];
        quant_chunk_fast_t<IN, FMT, STATS, false, false>(ch[j], r.s, r.y, r.T, valid, crow + c * 8u, h, st);
        if (XHAT && valid) store_xhat(a.xhat, a.xhat_dtype, (int64_t)row * cols + (int64_t)c * kChunk, h);
    }
}

// The scale of a whole tensor quantized over rows of it (per-tensor INT8 /
// FP8 on a contiguous tensor): every workgroup folds the absmax pre-pass's
// per-workgroup words (maximum and OR) and derives what the per-tensor flat
// kernel derives from them: s = alpha / Q, the FP32 fast path for a finite
// tensor with alpha in the statistics range, saturation possible when alpha
// exceeds T, exact zeros as flagged.  Workgroup 0 writes the scale.
template <int FMT, int NT>
__device__ __forceinline__ RowScale tensor_row_scale(const RowArgs& a) {
    __shared__ uint32_t s_pre[2][NT / 64][2];
    uint64_t w[kMaxGrid / NT];   // every load issued before the first use
#pragma unroll
    for (int k = 0; k < kMaxGrid / NT; ++k) {
        const int i = (int)threadIdx.x + k * NT;
        w[k] = i < a.amax_nwords ? a.amax_words[i] : 0u;
    }
    uint32_t m = 0u, fl = 0u;
#pragma unroll
    for (int k = 0; k < kMaxGrid / NT; ++k) {
        m = umax(m, (uint32_t)w[k]);
        fl |= (uint32_t)(w[k] >> 32);
    }
    bool nonfinite, zeros;
    const uint32_t bits = block_max_or<NT / 64>(m, (fl & 1u) != 0, nonfinite, s_pre[0]);
    block_max_or<NT / 64>(0u, (fl & 2u) != 0, zeros, s_pre[1]);
    const float alpha = as_f(bits);
    RowScale r;
    r.s = alpha / Fmt<FMT>::qmax;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.scale_out = r.s;
    r.fast = !nonfinite && stat_range(alpha);
    r.y = r.fast ? 1.0f / r.s : 0.f;
    r.T = r.fast ? sat_threshold<FMT>(r.s) : 0.f;
    r.sat = !r.fast || alpha > r.T;
    r.zeros = zeros;
    return r;
}

// Per-row INT8 / FP8: the next row streams into LDS while the current one
// is reduced, cast and stored.  XHAT: the x^ output is requested (a separate
// instantiation, so the other one carries no x^ code).
template <int IN, int FMT, int CPT, int NT, bool FULL, bool XHAT, bool STATS, bool TENSOR = false>
__global__ __launch_bounds__(NT) void k_quant_row(RowArgs a) {
    // Rows in flight per workgroup (LDS buffers).
    constexpr int DEPTH = kRowDepth<IN, CPT, NT, FULL>;
    __shared__ uint32_t s_red[3][NT / 64][2];
    __shared__ RowStage<IN, CPT, NT> stage[DEPTH];
    Stats st;
    RowScale rt{};
    if constexpr (TENSOR) rt = tensor_row_scale<FMT, NT>(a);
    const int32_t G = gridDim.x;
    const int64_t cols = (int64_t)a.cpr * kChunk;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int parity = 0, b = 0;
    int32_t row = blockIdx.x;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (row + d * G < a.rows) stage_row<IN, CPT, NT, FULL>(stage[d], a, row + d * G, wave);
    for (; row < a.rows; row += G, parity ^= 1, b = DEPTH > 1 ? b ^ 1 : 0) {
        Chunk<IN> ch[CPT];
        // With two buffers the copies of the next row (CPT * words per chunk
        // of them, all issued: FULL rows) were issued after this row's and
        // may stay in flight: the counter drains in issue order.
        if constexpr (DEPTH > 1) {
            if (row + G < a.rows) wait_staged_keep<CPT * ChunkWords<IN>::n>();
            else wait_staged();
        } else {
            wait_staged();
        }
        unstage_row<IN, CPT, NT, FULL>(stage[b], a, ch);
        wait_lds_reads();
        if (row + DEPTH * G < a.rows) stage_row<IN, CPT, NT, FULL>(stage[b], a, row + DEPTH * G, wave);
        RowScale r;
        if constexpr (TENSOR) {
            r = rt;
            // Keep the workgroup's waves on one row, as the per-row reduction
            // does: waves left to drift onto different rows issue their
            // copies interleaved with other rows' (BF16 65536 x 16384
            // per-tensor INT8: 655 us for this kernel without the barrier,
            // about 568 with it).
            lds_barrier();
        } else {
            r = row_scale<IN, FMT, CPT, NT>(ch, s_red, parity);
            if (threadIdx.x == 0) a.scales[row] = r.s;
        }
        uint8_t* crow = a.codes + (int64_t)row * cols;
        if (r.fast) {
            quant_row_fast<IN, FMT, CPT, NT, FULL, XHAT, STATS>(ch, a, row, r, crow, st);
        } else {
            quant_row_slow<IN, FMT, CPT, NT, FULL, XHAT, STATS>(a, row, r.s, crow, st);
        }
        if (STATS) st.fold();
    }
    if (STATS) write_partial<NT / 64>(st, a.sink);
}

// Rows longer than 2048 chunks: absmax pass, then a second
// pass that re-reads the row (from L2 for rows up to a few MiB).
template <int IN, int FMT, bool STATS>
__global__ __launch_bounds__(kThreads) void k_quant_row_long(RowArgs a) {
    constexpr float Q = Fmt<FMT>::qmax;
    __shared__ uint32_t s_red[3][kThreads / 64];
    const int tid = threadIdx.x;
    const int64_t cols = (int64_t)a.cpr * kChunk;
    Stats st;
    int parity = 0;
    for (int32_t row = blockIdx.x; row < a.rows; row += gridDim.x, parity ^= 1) {
        const int64_t base = (int64_t)row * a.ld;
        uint32_t m = 0;
        for (int c = tid; c < a.cpr; c += kThreads) {
            Chunk<IN> ch;
            ch.load(a.x, base + (int64_t)c * kChunk);
            ch.absmax(m);
        }
        uint32_t bits = block_max<kThreads / 64>(Chunk<IN>::absmax_bits(m), s_red[parity]);
        const bool nonfinite = bits >= kNonFinite;
        if (nonfinite) {   // Inf or NaN in the row: another pass for the finite absmax
            uint32_t f = 0;
            for (int c = tid; c < a.cpr; c += kThreads) {
                Chunk<IN> ch;
                ch.load(a.x, base + (int64_t)c * kChunk);
                f = umax(f, ch.absmax_finite());
            }
            bits = block_max<kThreads / 64>(f, s_red[2]);
        }
        const float alpha = as_f(bits);
        const float s = alpha / Q;
        if (tid == 0) a.scales[row] = s;
        const bool fast = !nonfinite && stat_range(alpha);
        const float y = fast ? 1.0f / s : 0.f;
        const float T = sat_threshold<FMT>(s);
        const bool sat = !fast || alpha > T;
        uint8_t* crow = a.codes + (int64_t)row * cols;
        // uniform trip count: lanes past the row end carry a zero chunk
        for (int c0 = 0; c0 < a.cpr; c0 += kThreads) {
            const int c = c0 + tid;
            const bool valid = c < a.cpr;
            Chunk<IN> ch;
            if (valid) ch.load(a.x, base + (int64_t)c * kChunk);
            else ch.zero();
            float h[8];
            quant_chunk_uniform<IN, FMT, STATS>(ch, s, y, fast, sat, T, true, valid, crow + (int64_t)c * kChunk, h, st);
            if (a.xhat && valid) store_xhat(a.xhat, a.xhat_dtype, (int64_t)row * cols + (int64_t)c * kChunk, h);
            if (STATS) st.fold();
        }
    }
    if (STATS) write_partial<kThreads / 64>(st, a.sink);
}

// ---------------------------------------------------------------------------
// Flat kernels: chunks of the [rows, cols] tensor in row-major order; each
// workgroup iteration covers kTileChunks consecutive chunks.
// ---------------------------------------------------------------------------
struct FlatGeom {
    const void* x;
    int64_t ld;
    uint32_t nchunks, cpr;
    int cpr_shift;   // log2(cpr) if cpr is a power of two, else -1
    int contiguous;  // ld == cols
    __device__ __forceinline__ int64_t elem(uint32_t g) const {
        if (contiguous) return (int64_t)g * kChunk;
        uint32_t row = cpr_shift >= 0 ? (g >> cpr_shift) : (g / cpr);
        return (int64_t)row * ld + (int64_t)(g - row * cpr) * kChunk;
    }
};

struct FlatArgs {
    FlatGeom geo;
    uint8_t* codes;
    void* scales;
    float* global_scale;
    void* xhat;
    int xhat_dtype;
    const uint64_t* amax_words;  // per-tensor INT8/FP8 and NVFP4: one word per pre-pass workgroup
    int32_t amax_nwords;         //   (absmax bits | flags << 32, flags 1 non-finite, 2 exact zero)
    const float* static_amax;    // static scaling: the caller's absmax instead of the pre-pass
    float* scale_out;            // where the per-tensor scale (or s_g) goes
    StatsSink sink;
    uint32_t rule;           // R_* scale-rule bits (MXFP4 exponent, NVFP4 block-scale rounding)
    uint8_t* shifts;         // asymmetric INT4: packed 4-bit shifts
};

// The functions below run on every lane of the wave (lanes past the end of
// the tensor carry a zero chunk, `valid` false); only stores are predicated,
// and the statistics are accumulated in wave-uniform control flow.

// Absmax of a block spread over G lanes (G = 2, 4, 16): bits of the finite
// maximum on every lane of the group; `nonfinite` if the block holds Inf/NaN.
template <int IN, int G>
__device__ __forceinline__ uint32_t unit_absmax(const Chunk<IN>& ch, bool& nonfinite, bool& chunk_zero) {
    uint32_t m, mn;
    ch.absmaxmin_word(m, mn);
    chunk_zero = Chunk<IN>::has_zero(mn);
    uint32_t bits = group_max<G>(Chunk<IN>::absmax_bits(m));
    nonfinite = bits >= kNonFinite;
    if (__ballot(nonfinite) != 0) {   // some block of the wave holds Inf or NaN
        const uint32_t f = group_max<G>(ch.absmax_finite());
        if (nonfinite) bits = f;
    }
    return bits;
}

// Flushed elements of a lane's chunks from its codes: every valid element
// is taken as a nonzero input, minus the nonzero codes (nz, accumulated per
// chunk); exact zero inputs are taken out by uncount_zero_inputs in the
// waves that hold one.
__device__ __forceinline__ void add_flushed(Stats& st, uint32_t nvalid, uint32_t nz) { st.lzf += 8u * nvalid - nz; }

// The chunks of a lane are cast one after another: pinned() hands out an
// opaque copy of a chunk (nothing that reads it can move above this point)
// and pin_sums() closes a chunk's statistics (nothing it feeds can move
// below).  Empty asm statements keep their program order, so the compiler
// cannot interleave the chunks, and each chunk's registers are released
// before the next one starts.
template <int IN> __device__ __forceinline__ Chunk<IN> pinned(const Chunk<IN>& ch) {
    Chunk<IN> c = ch;
#pragma unroll
    for (int k = 0; k < (int)(sizeof(c.w) / 4); ++k) asm volatile("" : "+v"(c.w[k]));
    return c;
}
__device__ __forceinline__ void pin_sums(Stats& st, uint32_t& nz) {
    asm volatile("" : "+v"(st.fx2), "+v"(st.fe2), "+v"(st.fae), "+v"(st.mae), "+v"(nz));
}

// Absmax over chunks [k0, k0 + K) of the lane: FP32 bits of the finite
// maximum, whether an Inf or NaN is present, whether an exact zero is.
template <int IN, int K>
__device__ __forceinline__ uint32_t lane_absmax(const Chunk<IN> (&ch)[kTileChunksPerThread], int k0, bool& nonfinite,
                                                bool& zero) {
    uint32_t m, mn;
    ch[k0].absmaxmin_word(m, mn);
#pragma unroll
    for (int k = 1; k < K; ++k) {
        uint32_t a, b;
        ch[k0 + k].absmaxmin_word(a, b);
        m = Chunk<IN>::hmax(m, a);
        mn = Chunk<IN>::hmin(mn, b);
    }
    const uint32_t bits = Chunk<IN>::absmax_bits(m);
    nonfinite = bits >= kNonFinite;
    zero = Chunk<IN>::has_zero(mn);
    return bits;
}

template <int IN, int K>
__device__ __forceinline__ uint32_t lane_absmax_finite(const Chunk<IN> (&ch)[kTileChunksPerThread], int k0) {
    uint32_t f = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) f = umax(f, ch[k0 + k].absmax_finite());
    return f;
}

// Store the 4 code words of the lane (one 16-byte store when all are valid).
__device__ __forceinline__ void store_words4(uint8_t* codes, uint32_t g0, uint32_t nvalid, const uint32_t (&w)[4]) {
    uint32_t* p = reinterpret_cast<uint32_t*>(codes) + g0;
    if (nvalid == 4) {
        const u4v o = {w[0], w[1], w[2], w[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<u4v*>(p));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if ((uint32_t)k < nvalid) __builtin_nontemporal_store(w[k], p + k);
    }
}

// First FP32 significand (bits 0..22) at or above 3*sqrt(2)/4 - 1: with
// A = m * 2^e, m in [1, 2), round(log2(A / 6)) = e - 3 + [m >= 3*sqrt(2)/4]
// (the half-way point 2^(k + 1/2) is irrational, so no FP32 value sits on it).
constexpr uint32_t kMxNearestMant = 0x07C3B7u;

// Unbiased E8M0 exponent of a block with finite absmax A = m * 2^e (bits of
// a positive float), before the bias and clamp:
//   default      floor(log2 A) - 2           = e - 2
//   R_MX_NEAREST round(log2(A / 6))          = e - 3 + [m >= 3*sqrt(2)/4]
//   R_MX_UP      ceil(log2(A / 6))           = e - 2 + [m > 3/2]
// For subnormal A the raw fraction stands in for m: every rule then lands
// below the clamp (e <= -127), whatever m is.
__device__ __forceinline__ int mx_exponent(uint32_t bits, uint32_t rule) {
    const int e = (bits >> 23) ? (int)(bits >> 23) - 127 : (31 - __clz((int)bits)) - 149;
    const uint32_t m = bits & 0x7FFFFFu;
    if (rule & R_MX_NEAREST) return e - 3 + (m >= kMxNearestMant ? 1 : 0);
    if (rule & R_MX_UP) return e - 2 + (m > 0x400000u ? 1 : 0);
    return e - 2;
}

// MXFP4: one block of 32 = the lane's 4 chunks.  E8M0 = clamp(E + 127, 0, 254)
// with E from mx_exponent.  g0 is the lane's first chunk (a multiple of 4),
// nvalid its chunks with data (0 or 4: the row length is a multiple of 32).
// The wave takes the fast body when every block of the wave is finite with
// its absmax in the FP32 statistics range: branch-free over the 4 chunks,
// with saturated elements and exact zeros counted first, in separate passes,
// by the waves that can hold them.  Otherwise every lane of the wave takes
// the general body: element by element from x in rolled loops (NaN codes
// patched, FP64 statistics), few registers for a rare case.
template <int IN, bool STATS, bool XHAT>
__device__ __forceinline__ void quant_lane_mx(const Chunk<IN> (&ch)[kTileChunksPerThread], uint32_t g0, uint32_t nvalid,
                                              const FlatArgs& a, Stats& st) {
    bool nonfinite, zero;
    uint32_t bits = lane_absmax<IN, 4>(ch, 0, nonfinite, zero);
    if (__ballot(nonfinite) != 0) {
        if (nonfinite) bits = lane_absmax_finite<IN, 4>(ch, 0);
    }
    int E = 0;
    if (bits) {
        E = mx_exponent(bits, a.rule) + 127;
        E = E < 0 ? 0 : (E > 254 ? 254 : E);
    }
    const float sc = E ? as_f((uint32_t)E << 23) : as_f(0x00400000u);   // 2^(E-127), exact
    if (nvalid != 0) static_cast<uint8_t*>(a.scales)[g0 >> 2] = (uint8_t)E;
    // Saturation without the quotient: |x / 2^(E-127)| > 6 exactly when
    // |x| > 6 * 2^(E-127) (both sides exact near 6).
    const float thr = 6.0f * sc;
    if (__ballot(nonfinite || !stat_range(as_f(bits))) == 0) {
        if (STATS && __ballot(zero) != 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) uncount_zero_inputs<IN>(st, ch[k], nvalid != 0);
        }
        uint32_t nz = 0, wq[4];
        // Saturated elements are counted with the cast in the waves where
        // some block can saturate (with the floor rule A / 2^(E-127) lies in
        // [4, 8): most blocks can).
        auto body = [&](auto count_sat) {
          constexpr bool SAT = decltype(count_sat)::value;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const Chunk<IN> cc = pinned(ch[k]);
            float x[8], h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = cc.get(i);
                if (STATS && SAT) st.nsat += __popcll(__ballot(__builtin_fabsf(x[i]) > thr));
            }
            uint32_t w = 0;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], sc, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], sc, 1);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], sc, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], sc, 3);
            const f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
            const f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
            const f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
            const f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
            h[0] = p0.x; h[1] = p0.y; h[2] = p1.x; h[3] = p1.y; h[4] = p2.x; h[5] = p2.y; h[6] = p3.x; h[7] = p3.y;
            if (STATS) {
                sums8<IN>(st, cc, x, h);
                nz += nonzero_nibbles(w);
                pin_sums(st, nz);
            }
            if (XHAT && nvalid != 0) store_xhat(a.xhat, a.xhat_dtype, (int64_t)(g0 + k) * kChunk, h);
            wq[k] = w;
          }
        };
        if (STATS && __ballot(as_f(bits) > thr) != 0) body(std::true_type{});
        else body(std::false_type{});
        store_words4(a.codes, g0, nvalid, wq);
        if (STATS) add_flushed(st, nvalid, nz);
    } else {
        uint32_t* codes32 = reinterpret_cast<uint32_t*>(a.codes);
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
            const bool valid = (uint32_t)c < nvalid;
            const int64_t e0 = valid ? a.geo.elem(g0 + c) : 0;
            uint32_t w = 0;
#pragma unroll 1
            for (int i = 0; i < 8; ++i) {
                const float x = valid ? load_elem<IN>(a.geo.x, e0 + i) : 0.f;
                // NaN has no E2M1 code: it maps to +0 (the convert would give +-6).
                uint32_t code = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, x, 0.f, sc, 0) & 0xFu;
                if (__builtin_isnan(x)) code = 0u;
                const float h = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, sc, 0)[0];
                w |= code << (4 * i);
                if (STATS) st.add1_slow(x, __builtin_fabsf(x) > thr, h);
                if (XHAT && valid) store_xhat1(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk + i, h);
            }
            if (valid) __builtin_nontemporal_store(w, codes32 + g0 + c);
        }
    }
}

// Smallest E4M3 code whose value is >= t (t >= 0, finite), capped at 448.
__device__ __forceinline__ uint32_t e4m3_ceil(float t) {
    if (t > 448.f) return 0x7Eu;
    uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xFFu;   // RNE
    return e4m3_value(c) < t ? c + 1u : c;
}

// Nearest E4M3 code to t (t >= 0, finite), ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
    if (t >= 448.f) return 0x7Eu;
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xFFu;
}

__device__ __forceinline__ uint32_t fp4_pack8(const float (&v)[8]) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
    return w;
}

__device__ __forceinline__ void fp4_unpack8(uint32_t w, float s, float (&h)[8]) {
    const f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    h[0] = s * p0.x; h[1] = s * p0.y; h[2] = s * p1.x; h[3] = s * p1.y;
    h[4] = s * p2.x; h[5] = s * p2.y; h[6] = s * p3.x; h[7] = s * p3.y;
}

// Per-launch NVFP4 constants: the global scale, its reciprocal, and for every
// E4M3 block code c the block scale s_g * value(c) with its correctly
// rounded reciprocal (LDS, filled once per workgroup).
struct NvConst {
    float s_g, y_g;
    bool g_fast;          // s_g >= kMarksteinMin: the block-scale quotient may use the correction
    bool rne;             // block scale to the nearest E4M3 instead of the next one up
    const f2v* tab;       // [128] {s_nv, 1 / s_nv}
};

// Block scale code: smallest E4M3 >= (A / 6) / s_g (k.rne: the nearest
// E4M3, ties to even, saturating at 448).  Both quotients come
// from the correction step when they are normal and the global scale is
// not tiny; other lanes (A tiny, block maxima far below the tensor's) take
// the two divisions.
__device__ __forceinline__ uint32_t nv_block_code(float A, const NvConst& k) {
    const float t1 = div_const<6>(A);
    const float t = markstein(t1, k.s_g, k.y_g);
    const bool exact = A == 0.f || (t1 >= kMarksteinMin && t >= kMarksteinMin && t <= 0x1p120f);
    float tt = t;
    if (__ballot(!(exact && k.g_fast)) != 0) {
        if (!(exact && k.g_fast)) tt = (A / 6.0f) / k.s_g;
    }
    return k.rne ? e4m3_rne(tt) : e4m3_ceil(tt);
}

// NVFP4: blocks of 16 = 2 chunks; the lane holds blocks (0, 1) and (2, 3) of
// its chunks.  The wave takes the fast body when every lane's blocks are
// finite with scales in the fast range (branch-free over the 4 chunks;
// saturated elements and exact zeros counted first, in separate passes, by
// the waves that can hold them); otherwise the general body, element by
// element from x in rolled loops (correctly rounded division, patches,
// FP64 statistics), which is exact for every lane.
template <int IN, bool STATS, bool XHAT>
__device__ __forceinline__ void quant_lane_nv(const Chunk<IN> (&ch)[kTileChunksPerThread], uint32_t g0, uint32_t nvalid,
                                              const NvConst& k, const FlatArgs& a, Stats& st) {
    bool nonfinite[2], zero[2];
    uint32_t bits[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) bits[b] = lane_absmax<IN, 2>(ch, 2 * b, nonfinite[b], zero[b]);
    if (__ballot(nonfinite[0] || nonfinite[1]) != 0) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
            if (nonfinite[b]) bits[b] = lane_absmax_finite<IN, 2>(ch, 2 * b);
    }
    uint32_t sb[2] = {0u, 0u};
    float s_nv[2] = {0.f, 0.f}, y[2] = {0.f, 0.f};
    if (k.s_g != 0.f) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sb[b] = nv_block_code(as_f(bits[b]), k);
            const f2v e = k.tab[sb[b]];
            s_nv[b] = e.x; y[b] = e.y;
        }
    }
    uint8_t* sc8 = static_cast<uint8_t*>(a.scales) + (g0 >> 1);
    if (nvalid == 4) *reinterpret_cast<uint16_t*>(sc8) = (uint16_t)(sb[0] | (sb[1] << 8));
    else if (nvalid >= 2) *sc8 = (uint8_t)sb[0];
    bool fast = true;
#pragma unroll
    for (int b = 0; b < 2; ++b) fast = fast && !nonfinite[b] && s_nv[b] >= kTinyScale && stat_range(as_f(bits[b]));
    if (__ballot(!fast) == 0) {
        if (STATS) {
            if (__ballot(can_saturate(as_f(bits[0]), s_nv[0], 6.f) || can_saturate(as_f(bits[1]), s_nv[1], 6.f)) != 0) {
                const float T0 = sat_threshold<F_NVFP4>(s_nv[0]), T1 = sat_threshold<F_NVFP4>(s_nv[1]);
#pragma unroll
                for (int c = 0; c < 4; ++c) count_above<IN>(st, ch[c], c < 2 ? T0 : T1);
            }
            if (__ballot(zero[0] || zero[1]) != 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) uncount_zero_inputs<IN>(st, ch[c], (uint32_t)c < nvalid);
            }
        }
        uint32_t nz = 0, wq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const Chunk<IN> cc = pinned(ch[c]);
            const float s = s_nv[c >> 1], yy = y[c >> 1];
            float x[8], v[8], h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = cc.get(i);
                v[i] = markstein(x[i], s, yy);
            }
            const uint32_t w = fp4_pack8(v);
            fp4_unpack8(w, s, h);
            if (STATS) {
                sums8<IN>(st, cc, x, h);
                nz += nonzero_nibbles(w);
                pin_sums(st, nz);
            }
            if (XHAT && (uint32_t)c < nvalid) store_xhat(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk, h);
            wq[c] = w;
        }
        store_words4(a.codes, g0, nvalid, wq);
        if (STATS) add_flushed(st, nvalid, nz);
    } else {
        uint32_t* codes32 = reinterpret_cast<uint32_t*>(a.codes);
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
            const bool valid = (uint32_t)c < nvalid;
            const float s = c < 2 ? s_nv[0] : s_nv[1];
            const int64_t e0 = valid ? a.geo.elem(g0 + c) : 0;
            uint32_t w = 0;
#pragma unroll 1
            for (int i = 0; i < 8; ++i) {
                const float x = valid ? load_elem<IN>(a.geo.x, e0 + i) : 0.f;
                const float v = (s == 0.f) ? 0.f : x / s;
                uint32_t code = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, v, 0.f, 1.0f, 0) & 0xFu;
                if (s == 0.f || __builtin_isnan(v)) code = 0u;
                const float h = s * __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0)[0];
                w |= code << (4 * i);
                if (STATS) st.add1_slow(x, __builtin_fabsf(v) > 6.f, h);
                if (XHAT && valid) store_xhat1(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk + i, h);
            }
            if (valid) __builtin_nontemporal_store(w, codes32 + g0 + c);
        }
    }
}

// 8 INT4 codes from t = v + 1.5 * 2^23 (the low nibble of each t is the
// two's-complement code, or the unsigned code of the asymmetric format):
// the low bytes of the even and of the odd elements are gathered into one
// word each, then the odd nibbles are shifted up and merged with one bit
// select (element 2j in bits 3:0 of byte j, element 2j+1 in bits 7:4).
__device__ __forceinline__ uint32_t int4_pack8(const float (&t)[8]) {
    const uint32_t e = __builtin_amdgcn_perm(as_u(t[2]), as_u(t[0]), 0x0c0c0400u) |
                       (__builtin_amdgcn_perm(as_u(t[6]), as_u(t[4]), 0x0c0c0400u) << 16);
    const uint32_t o = __builtin_amdgcn_perm(as_u(t[3]), as_u(t[1]), 0x0c0c0400u) |
                       (__builtin_amdgcn_perm(as_u(t[7]), as_u(t[5]), 0x0c0c0400u) << 16);
    return (e & 0x0F0F0F0Fu) | ((o << 4) & 0xF0F0F0F0u);
}

// INT4: groups of 128 = 16 chunks = 4 lanes; FP16 scale fp16(A / 7), saturated.
// rtab[f] = RN(1 / (1 + f / 1024)): the reciprocal of a normal FP16 scale
// 2^e (1 + f / 1024) is rtab[f] * 2^-e exactly (a power-of-two scaling of a
// normal binary32).  Fast body when every group of the wave is finite with
// a normal, unsaturated scale (saturated elements, |x| > T with T from
// sat_threshold, and exact zeros counted first in separate passes);
// otherwise the general body, element by element from x in rolled loops.
template <int IN, bool STATS, bool XHAT>
__device__ __forceinline__ void quant_lane_int4(const Chunk<IN> (&ch)[kTileChunksPerThread], uint32_t g0, uint32_t nvalid,
                                                const float* rtab, const FlatArgs& a, Stats& st) {
    bool nonfinite_l, zero;
    uint32_t bits = group_max<4>(lane_absmax<IN, 4>(ch, 0, nonfinite_l, zero));
    const bool nonfinite = group_max<4>(nonfinite_l ? 1u : 0u) != 0;
    if (__ballot(nonfinite) != 0) {
        const uint32_t f = group_max<4>(lane_absmax_finite<IN, 4>(ch, 0));
        if (nonfinite) bits = f;
    }
    float s32 = div_const<7>(as_f(bits));              // the correctly rounded A / 7 for every finite A
    // The FP32 quotient must be rounded to FP32 before the FP16 cast: without
    // this barrier the compiler fuses the last fma with the cast into one
    // fma with an FP16 result (a single rounding, different on FP16 ties).
    asm volatile("" : "+v"(s32));
    _Float16 hs = (_Float16)s32;                       // RNE
    uint16_t s16 = s32 > 65504.f ? (uint16_t)0x7BFF : __builtin_bit_cast(uint16_t, hs);
    const float sf = (float)__builtin_bit_cast(_Float16, s16);
    if (nvalid != 0 && (g0 & 15u) == 0) static_cast<uint16_t*>(a.scales)[g0 >> 4] = s16;
    // fast: finite inputs and a normal, unsaturated FP16 scale keep |x/sf| < 7.5
    // (and put A = 7 sf inside the FP32 statistics range)
    const bool fast = !nonfinite && sf >= 0x1p-14f && s32 <= 65504.f;
    if (__ballot(!fast) == 0) {
        if (STATS && __ballot(zero) != 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) uncount_zero_inputs<IN>(st, ch[c], (uint32_t)c < nvalid);
        }
        const int ex = (int)((s16 >> 10) & 0x1Fu) - 15;
        const float y = __builtin_amdgcn_ldexpf(rtab[s16 & 0x3FFu], -ex);
        // x^ = sf * q = fma(sf, t, -sf * kMagic): sf * kMagic and sf * q are
        // exact (11 + 2 and 11 + 3 significant bits), so the fma is exact.
        const float sfm = sf * kMagic;
        uint32_t nz = 0, wq[4];
        // Saturated elements, |v| > 7, counted from the quotient (the
        // division there) in the waves where some group can saturate: the
        // FP16 rounding of A / 7 puts A / sf above 7 in about half of them.
        auto body = [&](auto count_sat) {
            constexpr bool SAT = decltype(count_sat)::value;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const Chunk<IN> cc = pinned(ch[c]);
                float x[8], t[8], h[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[i] = cc.get(i);
                    const float v = markstein(x[i], sf, y);
                    if (STATS && SAT) st.nsat += __popcll(__ballot(__builtin_fabsf(v) > 7.f));
                    t[i] = v + kMagic;   // |v| <= 7.5: kMagic + RNE(v)
                    h[i] = __builtin_fmaf(sf, t[i], -sfm);
                }
                const uint32_t w = int4_pack8(t);
                if (STATS) {
                    sums8<IN>(st, cc, x, h);
                    nz += nonzero_nibbles(w);
                    pin_sums(st, nz);
                }
                if (XHAT && (uint32_t)c < nvalid) store_xhat(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk, h);
                wq[c] = w;
            }
        };
        if (STATS && __ballot(can_saturate(as_f(bits), sf, 7.f)) != 0) body(std::true_type{});
        else body(std::false_type{});
        store_words4(a.codes, g0, nvalid, wq);
        if (STATS) add_flushed(st, nvalid, nz);
    } else {
        uint32_t* codes32 = reinterpret_cast<uint32_t*>(a.codes);
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
            const bool valid = (uint32_t)c < nvalid;
            const int64_t e0 = valid ? a.geo.elem(g0 + c) : 0;
            uint32_t w = 0;
#pragma unroll 1
            for (int i = 0; i < 8; ++i) {
                const float x = valid ? load_elem<IN>(a.geo.x, e0 + i) : 0.f;
                const float v = (sf == 0.f) ? 0.f : x / sf;
                const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v), -7.f), 7.f);
                const int qi = __builtin_isnan(v) ? 0 : (int)q;   // via int: a zero code is +0
                const float h = sf * (float)qi;
                w |= ((uint32_t)qi & 0xFu) << (4 * i);
                if (STATS) st.add1_slow(x, __builtin_fabsf(v) > 7.f, h);
                if (XHAT && valid) store_xhat1(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk + i, h);
            }
            if (valid) __builtin_nontemporal_store(w, codes32 + g0 + c);
        }
    }
}

// Signed range over the finite elements of the lane's chunks (the rare path
// of groups holding Inf or NaN): FP32 bits of max(0, max x) and -min(0, min x).
template <int IN>
__device__ __forceinline__ void lane_range_finite(const Chunk<IN> (&ch)[kTileChunksPerThread], uint32_t& pos,
                                                  uint32_t& neg) {
    float hi = 0.f, nlo = 0.f;
#pragma unroll
    for (int c = 0; c < kTileChunksPerThread; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = ch[c].get(i);
            if (__builtin_isfinite(x)) {
                hi = __builtin_fmaxf(hi, x);
                nlo = __builtin_fmaxf(nlo, -x);
            }
        }
    }
    pos = as_u(hi) & 0x7FFFFFFFu;   // both are >= 0; drop the sign a max of +-0 may leave
    neg = as_u(nlo) & 0x7FFFFFFFu;
}

// The x-domain bound of RN(x / s) > q for an integer 0 <= q <= 15 and a
// scale s > 0: RN(x / s) > q exactly when x > RD((q + u) * s), with u half
// an ulp of q (q's significand is even, so the midpoint above q rounds down
// to q), and u = 2^-150 for q = 0 (the tie at half the smallest subnormal
// rounds to +0).  The FP64 product is exact (at most 25 + 24 bits).
__device__ __forceinline__ float above_int(int q, float s) {
    const double u = q == 0 ? 0x1p-150 : __builtin_ldexp(1.0, (31 - __clz(q)) - 24);
    return rd_to_float(((double)q + u) * (double)s);
}

// Elements of a chunk beyond the asymmetric grid: x > thi (positive side) or
// -x > tlo (negative side), compared on the integer images of an opaque
// copy of the raw words (signed for the positive side, where negative
// inputs compare below every bound; unsigned with the sign bit set for the
// negative side, where positive inputs compare below).  For BF16 the bounds
// are truncated to BF16, which keeps the comparisons exact.
template <int IN>
__device__ __forceinline__ void count_outside(Stats& st, const Chunk<IN>& ch, float thi, float tlo) {
    const uint32_t hb = as_u(thi), lb = as_u(tlo);
#pragma unroll
    for (int k = 0; k < (int)(sizeof(ch.w) / 4); ++k) {
        uint32_t w = ch.w[k];
        asm volatile("" : "+v"(w));
        if (IN == D_BF16) {
            const int ph = (int)(hb >> 16);
            const uint32_t nl = 0x8000u | (lb >> 16);
            const int w0 = (int)(int16_t)(w & 0xFFFFu), w1 = (int)(int16_t)(w >> 16);
            st.nsat += __popcll(__ballot(w0 > ph || (w & 0xFFFFu) > nl));
            st.nsat += __popcll(__ballot(w1 > ph || (w >> 16) > nl));
        } else {
            st.nsat += __popcll(__ballot((int)w > (int)hb || w > (0x80000000u | lb)));
        }
    }
}

// Asymmetric INT4 (the Triton post, Puzzle 12: x^ = sc * (w - sh) with
// unsigned 4-bit w and sh; the min-max encoder).  Groups of 128 = 16 chunks
// = 4 lanes.  Over the group's finite elements lo = min(0, min x) and
// hi = max(0, max x); sc = (hi - lo) / 15 (the largest float if that
// overflows); sh = RNE(-lo / sc) clamped to [0, 15];
// w = clamp(RNE(x / sc) + sh, 0, 15).  x / sc takes the correction step with
// y = RN(1 / sc): it equals the division except for quotients below 2^-20,
// which give the same code (checked on the CPU for every BF16 input of
// seeded BF16 group ranges).  A code equal to sh is exactly a zero x^, so
// flushed elements are counted from w ^ sh.  Saturated elements (x / sc
// above 15 - sh or below -sh) are counted from the quotient where both
// bounds are at least 1 in magnitude, else in the x domain (above_int).
template <int IN, bool STATS, bool XHAT>
__device__ __forceinline__ void quant_lane_int4zp(const Chunk<IN> (&ch)[kTileChunksPerThread], uint32_t g0,
                                                  uint32_t nvalid, const FlatArgs& a, Stats& st) {
    uint32_t p = 0, n = 0, mn = Chunk<IN>::kMagInit;
#pragma unroll
    for (int c = 0; c < kTileChunksPerThread; ++c) ch[c].range(p, n, mn);
    uint32_t pos, neg;
    Chunk<IN>::range_bits(p, n, pos, neg);
    const bool zero = Chunk<IN>::has_zero(mn);
    pos = group_max<4>(pos);
    neg = group_max<4>(neg);
    const bool nonfinite = pos >= kNonFinite || neg >= kNonFinite;
    if (__ballot(nonfinite) != 0) {
        uint32_t fp, fn;
        lane_range_finite<IN>(ch, fp, fn);
        fp = group_max<4>(fp);
        fn = group_max<4>(fn);
        if (nonfinite) { pos = fp; neg = fn; }
    }
    const float hi = as_f(pos), nlo = as_f(neg);          // lo = -nlo
    // (hi - lo) / 15: the constant-divisor correction is the division for
    // every finite span >= 0; an infinite span gives the largest float.
    const float span = hi + nlo;
    const float sc = span <= 0x1.fffffep127f ? div_const<15>(span) : 0x1.fffffep127f;
    const bool fast = !nonfinite && sc >= kTinyScale && stat_range(__builtin_fmaxf(hi, nlo));
    const bool wave_fast = __ballot(!fast) == 0;
    const float y = wave_fast ? 1.0f / sc : 0.f;
    // sh = RNE(nlo / sc) clamped to [0, 15]; on the fast path the corrected
    // quotient gives the same shift (checked on the CPU over seeded BF16
    // group ranges)
    int sh = 0;
    if (wave_fast) sh = (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(markstein(nlo, sc, y)), 0.f), 15.f);
    else if (sc != 0.f) sh = (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(nlo / sc), 0.f), 15.f);
    // the next group's shift, 4 lanes on (within the lane's row of 16; only
    // lanes 8k, whose next group is lanes 8k + 4 .. 8k + 7, use it)
    const int sh_next = __builtin_amdgcn_update_dpp(0, sh, 0x104, 0xF, 0xF, false);
    if (nvalid != 0) {
        if ((g0 & 15u) == 0) static_cast<float*>(a.scales)[g0 >> 4] = sc;
        if ((g0 & 31u) == 0) a.shifts[g0 >> 5] = (uint8_t)(sh | (sh_next << 4));
    }
    if (wave_fast) {
        // With 1 <= sh <= 14 in every group of the wave both bounds of the
        // grid, 15 - sh and -sh, are at least 1 in magnitude, where the
        // corrected quotient is the division: saturated elements are then
        // counted from it, v outside [-sh, 15 - sh] (about half the groups
        // hold one: hi / sc = 15 - sh + (sh - nlo / sc)).  A zero bound
        // (sh = 0 or 15) decides at the underflow threshold: there the
        // elements are compared with the exact x-domain bounds (above_int).
        const bool inner = __ballot(sh == 0 || sh == 15) == 0;
        if (STATS) {
            if (!inner) {
                const float thi = above_int(15 - sh, sc), tlo = above_int(sh, sc);
                if (__ballot(hi > thi || nlo > tlo) != 0) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) count_outside<IN>(st, ch[c], thi, tlo);
                }
            }
            if (__ballot(zero) != 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) uncount_zero_inputs<IN>(st, ch[c], (uint32_t)c < nvalid);
            }
        }
        const uint32_t shrep = (uint32_t)sh * 0x11111111u;
        // v is clamped to [-sh, 15 - sh] first (integer bounds, so rounding
        // the clamped value equals clamping the rounded one) and rounded to
        // q = RNE(vc) (ties to an even q, as the rounding happens before the
        // shift); t = q + (kMagic + sh) is exact and holds w in its low
        // nibble, and x^ = sc * q.  A q that rounds from a small negative vc
        // is -0: the x^ output takes q = (vc + kMagic) - kMagic, +0 there as
        // in x^ = sc * (w - sh); the statistics need no sign of zero.
        const float shf = (float)sh, magic_sh = kMagic + shf, vlo = -shf, vhi = 15.f - shf;
        uint32_t nz = 0, wq[4];
        auto body = [&](auto count_v) {
            constexpr bool COUNT_V = decltype(count_v)::value;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const Chunk<IN> cc = pinned(ch[c]);
                float x[8], t[8], h[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[i] = cc.get(i);
                    const float v = markstein(x[i], sc, y);
                    const float vc = __builtin_amdgcn_fmed3f(v, vlo, vhi);
                    if (STATS && COUNT_V) st.nsat += __popcll(__ballot(vc != v));
                    const float q = XHAT ? (vc + kMagic) - kMagic : __builtin_rintf(vc);
                    t[i] = q + magic_sh;
                    h[i] = sc * q;
                }
                const uint32_t w = int4_pack8(t);
                if (STATS) {
                    sums8<IN>(st, cc, x, h);
                    nz += nonzero_nibbles_full(w ^ shrep);   // w != sh: a nonzero x^
                    pin_sums(st, nz);
                }
                if (XHAT && (uint32_t)c < nvalid) store_xhat(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk, h);
                wq[c] = w;
            }
        };
        if (inner) body(std::true_type{});
        else body(std::false_type{});
        store_words4(a.codes, g0, nvalid, wq);
        if (STATS) add_flushed(st, nvalid, nz);
    } else {
        const float vhi = (float)(15 - sh), vlo = (float)(-sh);
        uint32_t* codes32 = reinterpret_cast<uint32_t*>(a.codes);
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
            const bool valid = (uint32_t)c < nvalid;
            const int64_t e0 = valid ? a.geo.elem(g0 + c) : 0;
            uint32_t w = 0;
#pragma unroll 1
            for (int i = 0; i < 8; ++i) {
                const float x = valid ? load_elem<IN>(a.geo.x, e0 + i) : 0.f;
                float v = 0.f;
                int wi = sh;
                if (sc != 0.f) {
                    v = x / sc;
                    if (!__builtin_isnan(v))
                        wi = (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(v) + (float)sh, 0.f), 15.f);
                }
                const float h = sc * (float)(wi - sh);
                w |= (uint32_t)wi << (4 * i);
                if (STATS) st.add1_slow(x, v > vhi || v < vlo, h);
                if (XHAT && valid) store_xhat1(a.xhat, a.xhat_dtype, (int64_t)(g0 + c) * kChunk + i, h);
            }
            if (valid) __builtin_nontemporal_store(w, codes32 + g0 + c);
        }
    }
}

// ---------------------------------------------------------------------------
// Flat tiles.  A workgroup iteration covers kTileChunks = 1024 consecutive
// chunks; for the block formats lane l of wave w owns the 4 consecutive
// chunks 256 w + 4 l + k of the tile (32 elements: one MXFP4 block, two
// NVFP4 blocks, a quarter of an INT4 group), for INT8 / FP8 per tensor the
// chunks 256 w + 64 k + l (FlatOwn).  The HBM -> LDS copies keep each instruction on 1 KiB of
// consecutive input: lane i of copy j fetches 16-byte word 64 j + unswz(i)
// of the wave's region, so word o lands in column swz(o mod 64) of row
// o / 64; a lane's reads of its own words then fall in distinct banks within
// every group of 8 lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t swz(uint32_t o) { return (o & ~7u) | ((o + (o >> 3)) & 7u); }
__device__ __forceinline__ uint32_t unswz(uint32_t i) { return (i & ~7u) | ((i - (i >> 3)) & 7u); }

// Per-tensor constants of the flat kernel.
struct FlatConst {
    float s, y, T;        // T: per-tensor saturation threshold in the x domain
    bool fast, sat, zeros;
    uint32_t amax_bits;   // the per-tensor absmax the scale came from
    NvConst nk;
    const float* rtab;
};

// Chunk ownership within a tile.  The block formats give lane l of wave w
// the 4 consecutive chunks 256 w + 4 l + k (whole blocks per lane or lane
// group).  INT8 / FP8 per tensor have no blocks: lane l owns chunks
// 256 w + 64 k + l, so the 8-byte code stores (and x^ stores) of a wave
// cover consecutive bytes, as in the per-row kernels.
template <int FMT> struct FlatOwn {
    static constexpr bool kInterleaved = FMT == F_INT8 || FMT == F_E4M3 || FMT == F_E5M2;
    static constexpr uint32_t kStride = kInterleaved ? 64u : 1u;   // chunk k of the lane is g0 + kStride * k
};

// One tile's worth of the lane's chunks (wd: its 16-byte words from LDS).
// FULL: every chunk of the tile holds data (no per-chunk validity selects).
// XHAT: the x^ output is written (a separate instantiation).
// CHECK (per-tensor INT8 / FP8 with a caller-supplied absmax): nothing is
// known of the data, so each wave takes the fast cast only when its inputs
// are finite, within the absmax (no clamping beyond the rounding of s) and
// not all below the FP32 statistics range; the exact-zero flag is the
// wave's own.
template <int IN, int FMT, bool STATS, bool FULL, bool CHECK, bool XHAT>
__device__ __forceinline__ void flat_lane(const u4v (&wd)[kTileChunksPerThread * ChunkWords<IN>::n], uint32_t g0,
                                          uint32_t nchunks, const FlatConst& k, const FlatArgs& a, Stats& st) {
    constexpr int W = ChunkWords<IN>::n;
    const uint32_t nvalid = FULL ? 4u : (g0 >= nchunks ? 0u : min(4u, nchunks - g0));
    Chunk<IN> ch[kTileChunksPerThread];
#pragma unroll
    for (int c = 0; c < kTileChunksPerThread; ++c) {
        const bool valid = FlatOwn<FMT>::kInterleaved ? (FULL || g0 + FlatOwn<FMT>::kStride * c < nchunks)
                                                      : (FULL || (uint32_t)c < nvalid);
        if (valid) ch[c].set(&wd[c * W], 1);
        else ch[c].zero();
    }
    if (FMT == F_MXFP4) {
        quant_lane_mx<IN, STATS, XHAT>(ch, g0, nvalid, a, st);
    } else if (FMT == F_NVFP4) {
        quant_lane_nv<IN, STATS, XHAT>(ch, g0, nvalid, k.nk, a, st);
    } else if (FMT == F_INT4) {
        quant_lane_int4<IN, STATS, XHAT>(ch, g0, nvalid, k.rtab, a, st);
    } else if (FMT == F_INT4ZP) {
        quant_lane_int4zp<IN, STATS, XHAT>(ch, g0, nvalid, a, st);
    } else {
        // INT8 / FP8 per tensor: the scale is the tensor's, the flags wave-uniform.
        bool fast = k.fast, zeros = k.zeros;
        if (CHECK) {
            bool nonfinite, zero;
            const uint32_t m = lane_absmax<IN, kTileChunksPerThread>(ch, 0, nonfinite, zero);
            fast = fast && __ballot(nonfinite || m > k.amax_bits) == 0 && __ballot(m >= as_u(kStatLo)) != 0;
            zeros = __ballot(zero) != 0;
        }
        if (fast) {
            // one branch-free body; saturated elements (tensors whose absmax
            // saturates) and exact zeros (waves holding one) counted first
            if (STATS && k.sat) {
#pragma unroll
                for (int c = 0; c < kTileChunksPerThread; ++c) count_above<IN>(st, ch[c], k.T);
            }
            if (STATS && zeros) {
#pragma unroll
                for (int c = 0; c < kTileChunksPerThread; ++c)
                    uncount_zero_inputs<IN>(st, ch[c], FULL || g0 + FlatOwn<FMT>::kStride * c < nchunks);
            }
#pragma unroll
            for (int c = 0; c < kTileChunksPerThread; ++c) {
                const uint32_t g = g0 + FlatOwn<FMT>::kStride * c;
                const bool valid = FULL || g < nchunks;
                float h[8];
                quant_chunk_fast_t<IN, FMT, STATS, false, false>(pinned(ch[c]), k.s, k.y, k.T, valid,
                                                                 a.codes + (int64_t)g * kChunk, h, st);
                if (STATS) {
                    uint32_t none = 0;
                    pin_sums(st, none);
                }
                if (XHAT && valid) store_xhat(a.xhat, a.xhat_dtype, (int64_t)g * kChunk, h);
            }
        } else {
            // element by element from x in rolled loops (correctly rounded
            // division, clamps, NaN codes, FP64 statistics)
            constexpr float Q = Fmt<FMT>::qmax;
#pragma unroll 1
            for (int c = 0; c < kTileChunksPerThread; ++c) {
                const uint32_t g = g0 + FlatOwn<FMT>::kStride * c;
                const bool valid = FULL || g < nchunks;
                const int64_t e0 = valid ? a.geo.elem(g) : 0;
                uint32_t w0 = 0, w1 = 0;
#pragma unroll 1
                for (int i = 0; i < 8; ++i) {
                    const float x = valid ? load_elem<IN>(a.geo.x, e0 + i) : 0.f;
                    float v, h;
                    const uint32_t code = cast1_slow<FMT>(x, k.s, v, h);
                    if (i < 4) w0 |= code << (8 * i);
                    else w1 |= code << (8 * (i - 4));
                    if (STATS) st.add1_slow(x, __builtin_fabsf(v) > Q, h);
                    if (XHAT && valid) store_xhat1(a.xhat, a.xhat_dtype, (int64_t)g * kChunk + i, h);
                }
                if (valid) {
                    const u2v o = {w0, w1};
                    __builtin_nontemporal_store(o, reinterpret_cast<u2v*>(a.codes + (int64_t)g * kChunk));
                }
            }
        }
    }
}

template <int IN, int FMT, bool STATS, bool CHECK, bool XHAT>
__global__ __launch_bounds__(kThreads) void k_quant_flat(FlatArgs a) {
    constexpr int W = ChunkWords<IN>::n;
    constexpr int NW = kTileChunksPerThread * W;      // 16-byte words per lane = copies per wave and tile
    static_assert(kTileChunksPerThread == 4, "lane layout assumes 4 chunks per lane");
    Stats st;
    const uint32_t ntiles = (a.geo.nchunks + kTileChunks - 1) / kTileChunks;
    // Tiles in flight per workgroup (LDS buffers): for BF16 INT4 and NVFP4
    // two with statistics and three without, one elsewhere.  Measured on BF16
    // 65536 x 16384: without statistics a third buffer takes INT4 from 491 to
    // 459 us (28672 x 8192: 105 -> 99 us), with statistics it costs 10 us (the
    // statistics kernels are bound by their VALU work, and 48 KB of LDS per
    // workgroup leaves 3 resident instead of 4); a second buffer slows the
    // MXFP4 and per-tensor kernels with statistics (513 -> 538 and 914 ->
    // 966 us).  FP32 tiles are twice as large.
    constexpr int DEPTH = IN == D_BF16 && (FMT == F_INT4 || FMT == F_NVFP4) ? (STATS ? 2 : 3) : 1;
    __shared__ Stage<NW> stage[DEPTH];
    const uint32_t lane = threadIdx.x & 63u;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t dlane = unswz(lane);
    const uint32_t esize = IN == D_BF16 ? 2u : 4u;
    auto stage_tile = [&](uint32_t tile, Stage<NW>& buf) {
        const uint32_t base = tile * kTileChunks + 256u * wave;
        if (a.geo.contiguous) {
            // word ow of the wave's region is the (base * W + ow)-th 16-byte word of x
            const char* wp = static_cast<const char*>(a.geo.x) + (size_t)base * W * 16u;
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const uint32_t ow = 64u * j + dlane;
                if (base + ow / W < a.geo.nchunks) dma_word(wp + ow * 16u, &buf[j][64 * wave]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const uint32_t ow = 64u * j + dlane;                // word of the wave's region
                const uint32_t c = base + ow / W;
                if (c < a.geo.nchunks)
                    dma_word(static_cast<const char*>(a.geo.x) + a.geo.elem(c) * esize + 16u * (ow % W), &buf[j][64 * wave]);
            }
        }
    };
    const uint32_t G = gridDim.x;
    // Per-tensor quantities (uniform over the grid): from the caller's absmax
    // (static scaling) or from the pre-pass's per-workgroup words, folded
    // here by every workgroup; workgroup 0 writes the scale.  A NaN,
    // negative or infinite caller absmax is taken as 0 and -0 as +0; nothing
    // is known of the data then (the per-tensor INT8 / FP8 kernel checks it
    // per wave), so the exact-zero flag is set.
    float s = 0.f, y = 0.f, T = 0.f;
    bool fast = false, sat = true, zeros = true;
    uint32_t amax_bits = 0u;
    if (FMT == F_INT8 || FMT == F_E4M3 || FMT == F_E5M2 || FMT == F_NVFP4) {
        constexpr float qdiv = FMT == F_INT8 ? 127.f : FMT == F_E4M3 ? 448.f : FMT == F_E5M2 ? 57344.f : 2688.f;
        bool nonfinite = false;
        if (a.static_amax) {
            float am = *a.static_amax;
            am = (am >= 0.f && am <= 0x1.fffffep127f) ? __builtin_fabsf(am) : 0.f;
            amax_bits = as_u(am);
        } else {
            __shared__ uint32_t s_pre[2][kThreads / 64][2];
            // Plain loads: the words were stored by the previous kernel on the
            // stream, and every workgroup reads the same 16 KB, so they are
            // served from L2 after the first.  All issued before the first use.
            uint64_t w[kMaxGrid / kThreads];
#pragma unroll
            for (int k = 0; k < kMaxGrid / kThreads; ++k) {
                const int i = (int)threadIdx.x + k * kThreads;
                w[k] = i < a.amax_nwords ? a.amax_words[i] : 0u;
            }
            uint32_t m = 0u, fl = 0u;
#pragma unroll
            for (int k = 0; k < kMaxGrid / kThreads; ++k) {
                m = umax(m, (uint32_t)w[k]);
                fl |= (uint32_t)(w[k] >> 32);
            }
            amax_bits = block_max_or<kThreads / 64>(m, (fl & 1u) != 0, nonfinite, s_pre[0]);
            block_max_or<kThreads / 64>(0u, (fl & 2u) != 0, zeros, s_pre[1]);
        }
        s = as_f(amax_bits) / qdiv;
        if (blockIdx.x == 0 && threadIdx.x == 0) *a.scale_out = s;
        const float alpha = as_f(amax_bits);
        fast = !nonfinite && stat_range(alpha);
        if constexpr (FMT == F_INT8 || FMT == F_E4M3 || FMT == F_E5M2) {
            if (fast) {
                y = 1.0f / s;
                T = sat_threshold<FMT>(s);
                sat = alpha > T;
            }
        }
    }
    // Reciprocal tables, filled once per workgroup with correctly rounded divisions.
    __shared__ f2v s_nvtab[FMT == F_NVFP4 ? 128 : 1];
    __shared__ float s_rtab[FMT == F_INT4 ? 1024 : 1];
    NvConst nk;
    nk.s_g = s; nk.y_g = 0.f; nk.g_fast = false; nk.rne = (a.rule & R_NV_RNE) != 0; nk.tab = s_nvtab;
    if (FMT == F_NVFP4) {
        if (s != 0.f) {
            nk.y_g = 1.0f / s;
            nk.g_fast = s >= kMarksteinMin;
        }
        if (threadIdx.x < 128) {
            const float sn = s * e4m3_value(threadIdx.x);
            f2v e;
            e.x = sn;
            e.y = sn > 0.f ? 1.0f / sn : 0.f;
            s_nvtab[threadIdx.x] = e;
        }
        __syncthreads();
    }
    if (FMT == F_INT4) {
        for (int f = threadIdx.x; f < 1024; f += kThreads) s_rtab[f] = 1.0f / (1.0f + (float)f * 0x1p-10f);
        __syncthreads();
    }
    // The first tiles are copied only now: issued before the prologue above,
    // the compiler's waits in the loop below came out differently (measured on
    // BF16 65536 x 16384 NVFP4: 10 us slower with statistics, 24 us faster
    // without).
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (blockIdx.x + d * G < ntiles) stage_tile(blockIdx.x + d * G, stage[d]);
    FlatConst fk;
    fk.s = s; fk.y = y; fk.T = T; fk.fast = fast; fk.sat = sat; fk.zeros = zeros; fk.nk = nk; fk.rtab = s_rtab;
    fk.amax_bits = (FMT == F_INT8 || FMT == F_E4M3 || FMT == F_E5M2) ? amax_bits : 0u;
    const uint32_t full_tiles = a.geo.nchunks / kTileChunks;
    int b = 0;
    for (uint32_t tile = blockIdx.x; tile < ntiles; tile += G, b = b + 1 < DEPTH ? b + 1 : 0) {
        // the lane's first chunk, and its words of the wave's region in LDS
        const uint32_t g0 = tile * kTileChunks + 256u * wave + (FlatOwn<FMT>::kInterleaved ? lane : 4u * lane);
        // This tile's copies have landed once at most the (DEPTH - 1) * NW
        // copies of the next tiles, issued after them, are outstanding
        // (memory operations of a wave complete in issue order); a next tile
        // that is not full may have been issued with fewer copies: then wait
        // for all.
        if constexpr (DEPTH > 1) {
            if (tile + (DEPTH - 1) * G < full_tiles) wait_staged_keep<(DEPTH - 1) * NW>();
            else wait_staged();
        } else {
            wait_staged();
        }
        u4v wd[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t ow = FlatOwn<FMT>::kInterleaved ? W * (64u * (k / W) + lane) + k % W : NW * lane + k;
            wd[k] = stage[b][ow >> 6][64 * wave + swz(ow & 63u)];
        }
        wait_lds_reads();
        if (tile + DEPTH * G < ntiles) stage_tile(tile + DEPTH * G, stage[b]);
        if (tile < full_tiles) flat_lane<IN, FMT, STATS, true, CHECK, XHAT>(wd, g0, a.geo.nchunks, fk, a, st);
        else flat_lane<IN, FMT, STATS, false, CHECK, XHAT>(wd, g0, a.geo.nchunks, fk, a, st);
        if (STATS) st.fold();
    }
    if (STATS) write_partial<kThreads / 64>(st, a.sink);
}

// ---------------------------------------------------------------------------
// Absmax pre-pass (per-tensor formats, the NVFP4 global scale, iq_amax).
// ---------------------------------------------------------------------------
// The result of the pre-pass and where it goes: the tensor header (info),
// the per-tensor scale alpha / qdiv or the NVFP4 global scale amax / 2688
// (scale_out), and the absmax itself (amax_out); each may be null.
struct AmaxSink {
    uint32_t* partials;   // one 64-bit word per workgroup: absmax bits | flags << 32
    uint32_t* ticket;     // arrival counters (kTicketBytes): zero at the start and at the end
    float qdiv;           // 0: no scale
    float* scale_out;
    float* amax_out;
};

// Each workgroup reduces its tiles to (absmax over finite elements, flags:
// 1 non-finite seen, 2 exact zero seen) in one word.  As the pre-pass of a
// quantize call (FOLD false) it stores the word and ends: the cast kernel,
// next on the stream, folds the words in each of its workgroups.  With FOLD
// (the absmax call, and empty tensors) the word is published with one
// device-scope atomic exchange and the workgroup counts its arrival; the
// last one folds all words (max and OR, order-free) and writes the results.
template <int IN, bool FOLD>
__global__ __launch_bounds__(kThreads) void k_amax(FlatGeom geo, AmaxSink sink) {
    __shared__ uint32_t s_red[2][kThreads / 64][2];
    __shared__ uint32_t s_last;
    const uint32_t ntiles = (geo.nchunks + kTileChunks - 1) / kTileChunks;
    uint32_t m = 0, raw = 0, mn = 0xFFFFFFFFu;
    for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        Chunk<IN> ch[kTileChunksPerThread];
        bool valid[kTileChunksPerThread];
#pragma unroll
        for (int j = 0; j < kTileChunksPerThread; ++j) {
            uint32_t g = tile * kTileChunks + j * kThreads + threadIdx.x;
            valid[j] = g < geo.nchunks;
            if (valid[j]) ch[j].load(geo.x, geo.elem(g));
            else ch[j].zero();
        }
#pragma unroll
        for (int j = 0; j < kTileChunksPerThread; ++j) {
            m = umax(m, ch[j].absmax_finite());
            uint32_t wx, wn;
            ch[j].absmaxmin_word(wx, wn);
            raw = Chunk<IN>::hmax(raw, wx);
            if (valid[j]) mn = Chunk<IN>::hmin(mn, wn);
        }
    }
    bool nonfinite, zeros;
    const uint32_t bits = block_max_or<kThreads / 64>(m, Chunk<IN>::absmax_bits(raw) >= kNonFinite, nonfinite, s_red[0]);
    block_max_or<kThreads / 64>(0u, Chunk<IN>::has_zero(mn), zeros, s_red[1]);
    const uint64_t word = (uint64_t)bits | ((uint64_t)((nonfinite ? 1u : 0u) | (zeros ? 2u : 0u)) << 32);
    if (!FOLD) {
        // The cast kernel launched next on the stream folds the words itself.
        if (threadIdx.x == 0) reinterpret_cast<uint64_t*>(sink.partials)[blockIdx.x] = word;
        return;
    }
    if (threadIdx.x == 0) {
        const uint64_t old = __hip_atomic_exchange(reinterpret_cast<uint64_t*>(sink.partials) + blockIdx.x, word,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(old) : "memory");   // performed before the ticket
        s_last = arrive_last(sink.ticket) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last == 0) return;
    uint32_t fm = 0, ff = 0;
    uint64_t w[kMaxGrid / kThreads];   // every load issued before the first use
#pragma unroll
    for (int k = 0; k < kMaxGrid / kThreads; ++k) {
        const int i = (int)threadIdx.x + k * kThreads;
        w[k] = __hip_atomic_load(reinterpret_cast<const uint64_t*>(sink.partials) + (i < (int)gridDim.x ? i : 0),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int k = 0; k < kMaxGrid / kThreads; ++k) {
        if ((int)threadIdx.x + k * kThreads >= (int)gridDim.x) continue;
        fm = umax(fm, (uint32_t)w[k]);
        ff |= (uint32_t)(w[k] >> 32);
    }
    bool any_nonfinite, any_zero;
    fm = block_max_or<kThreads / 64>(fm, (ff & 1u) != 0, any_nonfinite, s_red[0]);
    block_max_or<kThreads / 64>(0u, (ff & 2u) != 0, any_zero, s_red[1]);
    if (threadIdx.x == 0) {
        if (sink.scale_out) *sink.scale_out = sink.qdiv > 0.f ? as_f(fm) / sink.qdiv : 0.f;
        if (sink.amax_out) *sink.amax_out = as_f(fm);
    }
}

// Statistics of an empty tensor: n = 0 and every sum zero.
__global__ __launch_bounds__(64) void k_empty_stats(StatsOut* out) {
    if (threadIdx.x == 0) {
        StatsOut o = {};
        *out = o;
    }
}

// ---------------------------------------------------------------------------
// Dequantize: codes + scales -> x^ (FP32 or BF16), x^ = s * decode(q).
// ---------------------------------------------------------------------------
struct DeqArgs {
    uint32_t nchunks, cpr;
    int cpr_shift;
    const uint8_t* codes;
    const void* scales;
    const float* global_scale;
    const uint8_t* shifts;
    void* xhat;
    int xhat_dtype;
    int per_tensor;
};

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequant(DeqArgs a) {
    const uint32_t ntiles = (a.nchunks + kTileChunks - 1) / kTileChunks;
    for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
#pragma unroll
        for (int j = 0; j < kTileChunksPerThread; ++j) {
            const uint32_t g = tile * kTileChunks + j * kThreads + threadIdx.x;
            if (g >= a.nchunks) continue;
            float h[8];
            if (FMT == F_INT8 || FMT == F_E4M3 || FMT == F_E5M2) {
                const uint32_t row = a.per_tensor ? 0u : (a.cpr_shift >= 0 ? g >> a.cpr_shift : g / a.cpr);
                const float s = static_cast<const float*>(a.scales)[row];
                u2v c = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(a.codes) + g);
                if (FMT == F_INT8) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        int q = (int)(int8_t)(((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFFu);
                        h[i] = s * (float)q;
                    }
                } else {
                    f2v d0 = fp8_unpack2<FMT, false>(c.x), d1 = fp8_unpack2<FMT, true>(c.x);
                    f2v d2 = fp8_unpack2<FMT, false>(c.y), d3 = fp8_unpack2<FMT, true>(c.y);
                    h[0] = s * d0.x; h[1] = s * d0.y; h[2] = s * d1.x; h[3] = s * d1.y;
                    h[4] = s * d2.x; h[5] = s * d2.y; h[6] = s * d3.x; h[7] = s * d3.y;
                }
            } else {
                const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.codes) + g);
                if (FMT == F_MXFP4) {
                    const uint32_t E = static_cast<const uint8_t*>(a.scales)[g >> 2];
                    const float sc = E ? as_f(E << 23) : as_f(0x00400000u);
                    f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
                    f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
                    f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
                    f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
                    h[0] = p0.x; h[1] = p0.y; h[2] = p1.x; h[3] = p1.y; h[4] = p2.x; h[5] = p2.y; h[6] = p3.x; h[7] = p3.y;
                    if (E == 255u) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) h[i] = __builtin_nanf("");
                    }
                } else if (FMT == F_NVFP4) {
                    const uint32_t sb = static_cast<const uint8_t*>(a.scales)[g >> 1];
                    const float s_nv = a.global_scale[0] * e4m3_value(sb);
                    f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
                    f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
                    f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
                    f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
                    h[0] = s_nv * p0.x; h[1] = s_nv * p0.y; h[2] = s_nv * p1.x; h[3] = s_nv * p1.y;
                    h[4] = s_nv * p2.x; h[5] = s_nv * p2.y; h[6] = s_nv * p3.x; h[7] = s_nv * p3.y;
                } else if (FMT == F_INT4ZP) {
                    const float sc = static_cast<const float*>(a.scales)[g >> 4];
                    const int sh = (int)((a.shifts[g >> 5] >> (4u * ((g >> 4) & 1u))) & 0xFu);
#pragma unroll
                    for (int i = 0; i < 8; ++i) h[i] = sc * (float)((int)((w >> (4 * i)) & 0xFu) - sh);
                } else {
                    const uint16_t s16 = static_cast<const uint16_t*>(a.scales)[g >> 4];
                    const float sf = (float)__builtin_bit_cast(_Float16, s16);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        int q = (int)((w >> (4 * i)) & 0xFu);
                        q = (q & 7) - (q & 8);
                        h[i] = sf * (float)q;
                    }
                }
            }
            store_xhat(a.xhat, a.xhat_dtype, (int64_t)g * kChunk, h);
        }
    }
}

// ---------------------------------------------------------------------------
// The Puzzle 12 consumer on the matrix cores:
//   z[j, k] = sum_g sc[j, g] * sum_{l in g} (w[j, l] - sh[j, g]) * x[k, l]
// (Triton post, Puzzle 12; x token-major).  Within a group of 128, w - sh is
// an integer in [-15, 15], exact in BF16, so v_mfma_f32_16x16x32_bf16 forms
// exact products of it and the BF16 activations, summed in FP32; each group's
// sum is scaled by sc and added with one fma.
// From 33 tokens on a workgroup computes a 128-row tile of z: 64 tokens with
// four waves of 64 x 32 (33 to 64 tokens), 128 tokens with four waves of
// 64 x 64, or 256 tokens with eight (4 x 4 MFMA tiles of 16 x 16 per 64 x 64
// wave tile); launch_zp_gemm picks the width.  Per group the activations
// and codes of the next group load into registers during the MFMAs (direct
// global-to-LDS copies were the bottleneck), then the activations are
// written and the weights dequantized into LDS, WN threads per row.  Both
// tiles keep 16-byte slot c of row r at c ^ (r & 15), so the fragment reads
// (16 rows, one 16-byte slot each) hit distinct banks.
// MFMA operand layout (16x16x32): lane l supplies row l % 16 of A and column
// l % 16 of B with the same 8 consecutive k (a fixed slice per l / 16), and
// receives D[4 (l / 16) + i][l % 16], i = 0..3.
// ---------------------------------------------------------------------------
constexpr int kGemmTile = 128;

struct ZpGemmArgs {
    const uint8_t* codes;    // [n0, K / 2]
    const float* scales;     // [n0, K / 128]
    const uint8_t* shifts;   // [n0, K / 256]
    const uint16_t* x;       // [n1, K] BF16
    float* z;                // [n0, n1]
    int32_t n0, n1, K;
    int32_t tiles_j, tiles_n, per_xcd;   // tile grid, work items per XCD slice
    uint32_t tiles;                      // tiles_j * tiles_n * ksplit (checked on the host)
    int32_t ksplit;                      // 1, or 2: k halves added atomically into a zeroed z
};

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// Tile (jb, nb) of GEMM work item idx.  The items of one XCD are
// consecutive, and the workgroups that XCD holds at once run consecutive
// items: walking GJ weight-row tiles of a token tile before the next token
// tile makes them share both operands in that XCD's L2, where row-major
// order (every token tile of one weight-row tile first) streams the whole
// activation matrix past each pair of weight tiles.  Measured at 2048 / 8192
// tokens against row-major order: FP4 GEMM (GJ 8) 116 -> 109 / 470 -> 390
// us, MXFP4 x BF16 (GJ 16) 292 -> 279 / 1160 -> 965 us, asymmetric INT4
// (GJ 16) 1210 -> 1151 / 5195 -> 5004 us; groups of 32 and 64 were slower
// for all three.  Unchanged up to 256 tokens.
template <uint32_t GJ>
__device__ __forceinline__ void gemm_tile_of(uint32_t idx, uint32_t tiles_j, uint32_t tiles_n, int& jb, int& nb) {
    const uint32_t gsize = GJ * tiles_n, grp = idx / gsize, first = grp * GJ;
    const uint32_t gj = min(tiles_j - first, GJ), in = idx - grp * gsize;
    jb = (int)(first + in % gj);
    nb = (int)(in / gj);
}
typedef float f4v __attribute__((ext_vector_type(4)));

// 8 weights (one code word, element i in bits 4i..4i+3) as BF16 w - sh.
// The even and the odd elements are masked into bytes once, each byte
// converts to float exactly, and w - sh (an integer in [-15, 15]) is exact
// in BF16: its upper half.  The asm keeps the compiler from splitting the
// masks back into one bit-field extract per element.
__device__ __forceinline__ u4v dequant8_bf16(uint32_t w, float sh) {
    uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    asm volatile("" : "+v"(ev), "+v"(od));
    float f[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f[2 * b] = (float)((ev >> (8 * b)) & 0xFFu) - sh;
        f[2 * b + 1] = (float)((od >> (8 * b)) & 0xFFu) - sh;
    }
    u4v o;
    o.x = __builtin_amdgcn_perm(as_u(f[1]), as_u(f[0]), 0x07060302u);
    o.y = __builtin_amdgcn_perm(as_u(f[3]), as_u(f[2]), 0x07060302u);
    o.z = __builtin_amdgcn_perm(as_u(f[5]), as_u(f[4]), 0x07060302u);
    o.w = __builtin_amdgcn_perm(as_u(f[7]), as_u(f[6]), 0x07060302u);
    return o;
}

// Few tokens (n1 <= 32): the weights are read once, so HBM and the
// dequantization bound the time, not the matrix cores.  A workgroup takes a
// stripe of 16 FR weight rows (FR = 2 fragments up to 8 tokens, 4 above,
// where one activation load then feeds twice the MFMAs) and 16 NT tokens;
// its 4 waves split the group
// pairs (wave w takes pairs w, w + 4, ...) and dequantize their codes in
// registers straight into MFMA operands (no LDS tile); the waves' partial sums
// meet in LDS at the end, added in wave order.
// The activations are operand A (rows = tokens) and the weights operand B
// (columns = weight rows): lane l dequantizes weight row 16 f + l % 16 and
// receives results of that same row (tokens 4 (l / 16) .. + 3), so its fold
// takes one scale per group.  For MFMA step q of group g lane l holds the k
// slice g * 128 + 32 (l / 16) + 8 q .. + 8: one code word of its 16-byte code
// load, and one 16-byte activation load per token tile.
// The codes of the next pair load while a pair computes; a pair's
// activations load just before (loads complete in order, so a wait for them
// leaves the codes in flight).  Scales and shift bytes come from LDS: read
// per lane from memory, 16 rows apart, they cost a fifth of the call.
// Rows past n0 and tokens past n1 read row n0 - 1 and token n1 - 1 instead:
// such lanes only feed outputs that are never stored, and no load is
// conditional.
template <int FR> struct GemvPair {
    u4v c[FR][2];      // codes [fragment][group of the pair]
};

// Scales and shift bytes of the workgroup's rows reach LDS in chunks of
// up to kGemvChunk pairs of groups, with coalesced loads (row-contiguous in
// memory), before the waves work through the chunk.  Rows are padded so the
// 16 rows that a wave's lanes read sit in distinct banks.
constexpr int kGemvChunk = 32;

// With one token tile and FR = 2, four waves per SIMD (at most 128
// registers, no spills) hold the whole grid of a 28672-row weight matrix at
// once: no second, mostly idle round; FR = 4 takes three.  A second register
// set of activations (one pair ahead) costs that occupancy and measured
// slower.
// X1 (a single token): the chunk's slice of the one activation row joins
// the scales in LDS (16 KB), so no activation load waits behind the codes.
template <int NT, bool X1, int FR>
__global__ __launch_bounds__(kThreads, NT == 1 ? (FR == 2 ? 4 : 3) : 1) void k_zp_gemv(ZpGemmArgs a) {
    constexpr int kRows = 16 * FR;
    static_assert(!X1 || NT == 1, "one token, one token tile");
    __shared__ f4v red[4][FR][NT][64];
    __shared__ float s_sc[kRows][2 * kGemvChunk + 1];
    __shared__ uint8_t s_sh[kRows][kGemvChunk + 4];
    __shared__ u4v s_x[X1 ? 2 * kGemvChunk * 16 : 1];
    const int j0 = (int)blockIdx.x * kRows, t0 = (int)blockIdx.y * 16 * NT;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int rr = lane & 15, h = lane >> 4;
    const int ng = a.K / 128, np = ng / 2;
    const uint8_t* crow[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
        const int64_t j = min(j0 + 16 * f + rr, a.n0 - 1);
        crow[f] = a.codes + j * (a.K / 2) + 16 * h;
    }
    const u4v* xr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t tok = min(t0 + 16 * nt + rr, a.n1 - 1);
        xr[nt] = reinterpret_cast<const u4v*>(a.x + tok * a.K + 32 * h);
    }
    auto load_pair = [&](int p, GemvPair<FR>& w) {
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            w.c[f][0] = *reinterpret_cast<const u4v*>(crow[f] + p * 128);
            w.c[f][1] = *reinterpret_cast<const u4v*>(crow[f] + p * 128 + 64);
        }
    };
    auto load_x = [&](int p, int pc, u4v (&xw)[2][NT][4]) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xw[e][nt][q] = X1 ? s_x[(2 * pc + e) * 16 + 4 * h + q] : xr[nt][(2 * p + e) * 16 + q];
    };
    f4v acc[FR][NT];
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[f][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    // pc: the pair's index within the staged chunk
    auto compute_pair = [&](int pc, const GemvPair<FR>& w, const u4v (&xp)[2][NT][4]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
            for (int f = 0; f < FR; ++f) {
                const int r = 16 * f + rr;
                const float sh = (float)((s_sh[r][pc] >> (4 * e)) & 0xFu);
                const float sc = s_sc[r][2 * pc + e];
                const uint32_t cw[4] = {w.c[f][e].x, w.c[f][e].y, w.c[f][e].z, w.c[f][e].w};
                f4v accg[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) accg[nt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf8v bw = __builtin_bit_cast(bf8v, dequant8_bf16(cw[q], sh));
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        accg[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, xp[e][nt][q]), bw,
                                                                           accg[nt], 0, 0, 0);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[f][nt][i] = __builtin_fmaf(sc, accg[nt][i], acc[f][nt][i]);
            }
        }
    };
    for (int p0 = 0; p0 < np; p0 += kGemvChunk) {
        const int p1 = min(np, p0 + kGemvChunk), cp = p1 - p0;
        __syncthreads();                         // the previous chunk's scales are no longer read
        for (int i = t; i < kRows * 2 * cp; i += kThreads) {
            const int r = i / (2 * cp), gg = i - r * (2 * cp);
            s_sc[r][gg] = a.scales[(int64_t)min(j0 + r, a.n0 - 1) * ng + 2 * p0 + gg];
        }
        for (int i = t; i < kRows * cp; i += kThreads) {
            const int r = i / cp, pp = i - r * cp;
            s_sh[r][pp] = a.shifts[(int64_t)min(j0 + r, a.n0 - 1) * np + p0 + pp];
        }
        if (X1) {
            const u4v* xg = reinterpret_cast<const u4v*>(a.x) + (int64_t)(2 * p0) * 16;
            for (int i = t; i < 2 * cp * 16; i += kThreads) s_x[i] = xg[i];
        }
        __syncthreads();
        if (p0 + wave < p1) {
            // the activations of a pair load before the next pair's codes, so
            // waiting for them leaves that prefetch in flight
            GemvPair<FR> pa, pb;
            u4v xw[2][NT][4];
            load_pair(p0 + wave, pa);
            for (int p = p0 + wave; p < p1; p += 8) {
                load_x(p, p - p0, xw);
                asm volatile("" ::: "memory");
                load_pair(min(p + 4, p1 - 1), pb);
                compute_pair(p - p0, pa, xw);
                load_x(min(p + 4, p1 - 1), min(p + 4, p1 - 1) - p0, xw);
                asm volatile("" ::: "memory");
                load_pair(min(p + 8, p1 - 1), pa);
                if (p + 4 < p1) compute_pair(p + 4 - p0, pb, xw);
            }
        }
    }
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave][f][nt][lane] = acc[f][nt];
    __syncthreads();
    // thread (part = t / 64, lane) sums the (fragment, token tile) pairs
    // congruent to part mod 4 and writes 4 tokens of row j0 + 16 f + lane % 16
    const int part = t >> 6;
#pragma unroll
    for (int fi = 0; fi < FR * NT; ++fi) {
        if (fi % 4 != part) continue;
        const int f = fi / NT, nt = fi % NT;
        const int j = j0 + 16 * f + rr;
        if (j >= a.n0) continue;
        const f4v v = ((red[0][f][nt][lane] + red[1][f][nt][lane]) + red[2][f][nt][lane]) + red[3][f][nt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * nt + 4 * h + i;
            if (tok < a.n1) a.z[(int64_t)j * a.n1 + tok] = v[i];
        }
    }
}

// Split-k epilogue for outputs whose rows do not start on 64-byte
// boundaries (n1 not a multiple of 16): each wave's 64 x 64 block of sums
// (rows mt 16 + 4 (lane / 16) + i, tokens nt 16 + lane % 16 of acc[mt][nt][i])
// goes through LDS, four waves at a time, and is added one row per atomic
// instruction: 64 floats, 256 contiguous bytes, where the direct form adds
// four 64-byte pieces of four rows and touches twice the cache lines.  The
// column swizzle (by row / 4) keeps the writes and the reads free of bank
// conflicts.  Called by every wave of the workgroup; blk needs 64 KB.
template <int NWAVES>
__device__ __forceinline__ void atomic_add_rows(const f4v (&acc)[4][4], float* blk, int wave, int lane, float* z,
                                                int32_t n0, int32_t n1, int row0, int tok0) {
    for (int w0 = 0; w0 < NWAVES; w0 += 4) {
        __syncthreads();
        float* mine = blk + (wave - w0) * 64 * 64;
        if (wave >= w0 && wave < w0 + 4) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        mine[(mt * 16 + 4 * (lane >> 4) + i) * 64 + ((nt * 16 + (lane & 15)) ^ ((lane >> 4) << 4))] =
                            acc[mt][nt][i];
        }
        __syncthreads();
        if (wave >= w0 && wave < w0 + 4) {
            const int tok = tok0 + lane;
            for (int r = 0; r < 64; ++r) {
                const int j = row0 + r;
                if (j < n0 && tok < n1)
                    unsafeAtomicAdd(z + (int64_t)j * n1 + tok, mine[r * 64 + (lane ^ (((r >> 2) & 3) << 4))]);
            }
        }
    }
}

// A tile of 128 weight rows x TNX tokens with NW waves in 2 rows of NW / 2
// (wave tiles 64 x TNX / (NW / 2)): 64 x 64 wave tiles for 128 and 256
// tokens (4 and 8 waves), 64 x 32 for 64 tokens (4 waves).  The
// dequantization of a weight tile is shared by all its tokens, so a wider
// tile spends fewer VALU cycles per MFMA.
// A grid too small to give every CU two groups in flight splits k in two
// halves (ksplit = 2): each work item sums its half and adds it atomically
// into z, which a fill kernel zeroed first.  With exactly two addends on a
// +0 start the sum is a + b, rounded once, in either order, so the result
// does not depend on which half lands first.
template <int TNX, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_zp_gemm(ZpGemmArgs a) {
    constexpr int kTN = TNX;                 // tokens per tile
    constexpr int NTH = 64 * NW;             // threads
    constexpr int WT = NW / 2;               // waves along the tokens (2 along the rows)
    constexpr int NB = kTN / WT / 16;        // 16-token MFMA blocks per wave
    constexpr int TPR = NTH / kGemmTile;     // staging threads per weight row
    constexpr int kWords = 4 / TPR;          // 16-byte code words per thread and group
    constexpr int kX = kTN * 16 / NTH;       // 16-byte activation words per thread and group
    __shared__ u4v tiles[(kGemmTile + kTN) * 16];
    u4v* const sA = tiles;                   // weights (w - sh) BF16, swizzled rows of 128
    u4v* const sB = tiles + kGemmTile * 16;  // activations BF16, same layout
    __shared__ float sS[kGemmTile];          // the group's scales of the tile's rows
    // Work items of one XCD slice are consecutive (gemm_tile_of).
    const uint32_t b = blockIdx.x;
    const uint32_t idx = (b & 7u) * (uint32_t)a.per_xcd + (b >> 3);
    if (idx >= a.tiles) return;
    const uint32_t tile = idx / (uint32_t)a.ksplit;
    const int half = (int)(idx % (uint32_t)a.ksplit);
    int jb, nb;
    gemm_tile_of<16>(tile, (uint32_t)a.tiles_j, (uint32_t)a.tiles_n, jb, nb);
    const int j0 = jb * kGemmTile, t0 = nb * kTN;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WT, wn = wave % WT;
    const int ng = a.K / 128;
    // the groups [g0, g1) of this work item's part of k
    const int g0 = (int)((int64_t)half * ng / a.ksplit), g1 = (int)((int64_t)(half + 1) * ng / a.ksplit);
    const int ldc = a.K / 2;             // code bytes per weight row
    f4v acc[4][NB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) acc[mt][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    // staging: thread t moves 16-byte slot t & 15 of token rows t / 16 + NTH / 16 i
    // (i < kX), the codes of weight row t / TPR (32 kWords from dp * 32 kWords)
    // with the row's shift byte, and (t < 128) the scale of row t
    const int xr0 = t >> 4, xs = t & 15;
    const uint16_t* gx[kX];
    int lx[kX];
#pragma unroll
    for (int i = 0; i < kX; ++i) {
        const int row = xr0 + NTH / 16 * i;
        gx[i] = a.x + (int64_t)min(t0 + row, a.n1 - 1) * a.K + xs * 8;
        lx[i] = row * 16 + (xs ^ (row & 15));
    }
    const int dr = t / TPR, dp = t % TPR;
    const int64_t dj = min(j0 + dr, a.n0 - 1);
    const u4v* gc = reinterpret_cast<const u4v*>(a.codes + dj * ldc + dp * 16 * kWords);
    const uint8_t* gsh = a.shifts + dj * (ng / 2);
    const float* gsc = a.scales + (int64_t)min(j0 + (t & (kGemmTile - 1)), a.n0 - 1) * ng;
    u4v rx[kX], rc[kWords];
    uint32_t rsb = 0;
    float rsc = 0.f;
    auto load_group = [&](int g) {
#pragma unroll
        for (int i = 0; i < kX; ++i) rx[i] = *reinterpret_cast<const u4v*>(gx[i] + g * 128);
#pragma unroll
        for (int v = 0; v < kWords; ++v) rc[v] = gc[g * 4 + v];
        rsb = gsh[g >> 1];
        if (t < kGemmTile) rsc = gsc[g];
    };
    if (g0 < g1) load_group(g0);
    for (int g = g0; g < g1; ++g) {
        __syncthreads();                     // every wave is done with the previous group's tiles
#pragma unroll
        for (int i = 0; i < kX; ++i) sB[lx[i]] = rx[i];
        const float sh = (float)((rsb >> (4 * (g & 1))) & 0xFu);
#pragma unroll
        for (int v = 0; v < kWords; ++v) {
            const uint32_t cw[4] = {rc[v].x, rc[v].y, rc[v].z, rc[v].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sA[dr * 16 + ((dp * 4 * kWords + 4 * v + q) ^ (dr & 15))] = dequant8_bf16(cw[q], sh);
        }
        if (t < kGemmTile) sS[t] = rsc;
        if (g + 1 < g1) load_group(g + 1);   // lands during this group's MFMAs
        lds_barrier();
        f4v accg[4][NB];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) accg[mt][nt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int slot = 4 * s + (lane >> 4);
            bf8v af[4], bfr[NB];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int r = wm * 64 + mt * 16 + (lane & 15);
                af[mt] = __builtin_bit_cast(bf8v, sA[r * 16 + (slot ^ (r & 15))]);
            }
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int r = wn * (kTN / WT) + nt * 16 + (lane & 15);
                bfr[nt] = __builtin_bit_cast(bf8v, sB[r * 16 + (slot ^ (r & 15))]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
                    accg[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], accg[mt][nt], 0, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sc = sS[wm * 64 + mt * 16 + 4 * (lane >> 4) + i];
#pragma unroll
                for (int nt = 0; nt < NB; ++nt) acc[mt][nt][i] = __builtin_fmaf(sc, accg[mt][nt][i], acc[mt][nt][i]);
            }
    }
    if constexpr (NB == 4) {
        static_assert((kGemmTile + kTN) * 16 * 16 >= 4 * 64 * 64 * 4, "four 64 x 64 blocks fit in the tiles");
        if (a.ksplit > 1 && (a.n1 & 15)) {
            atomic_add_rows<NW>(acc, reinterpret_cast<float*>(tiles), wave, lane, a.z, a.n0, a.n1, j0 + wm * 64,
                                t0 + wn * 64);
            return;
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + wm * 64 + mt * 16 + 4 * (lane >> 4) + i;
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int tok = t0 + wn * (kTN / WT) + nt * 16 + (lane & 15);
                if (j < a.n0 && tok < a.n1) {
                    if (a.ksplit > 1) unsafeAtomicAdd(a.z + (int64_t)j * a.n1 + tok, acc[mt][nt][i]);
                    else a.z[(int64_t)j * a.n1 + tok] = acc[mt][nt][i];
                }
            }
        }
}

// ---------------------------------------------------------------------------
// FP4 GEMM over two MXFP4 operands on gfx950's block-scaled matrix cores:
//   z[j, t] = sum_k xw[j, k] * xa[t, k],  x = 2^(E - 127) * e2m1(code)
// (low-precision post, "FP4 / MXFP4 / NVFP4": the MXFP4 value of a code).
// v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands takes, per lane, 32
// codes (16 bytes) of row l % 16 at k block l / 16 of a 128-deep step, and
// one E8M0 scale byte for exactly those 32: the MXFP4 storage layout itself
// (16 contiguous code bytes and one scale byte per block).  The products
// are exact and summed in FP32, so no dequantization or per-block fold runs
// on the VALU.
// A workgroup computes a TM x TN tile of z with 4 waves: 2 x 2 of 64 x TN/2
// for TM = 128, 1 x 4 of 64 x TN/4 for TM = 64 (small grids).  Per k step
// the codes of both operands (64 bytes per row) and their scale words (one
// 32-bit word of 4 E8M0 bytes per row) are staged through registers into a
// double-buffered LDS tile: step k + 2 loads into registers while step k
// computes, and is written to LDS during step k + 1 after that step's
// operands have been read.  (Direct global-to-LDS copies of these half-line
// rows measured about 3x slower; k_mx_gemm_dma below copies whole lines.)
// One LDS-only barrier per step: it must not wait for the
// register loads in flight.  Code rows are 4 slots of 16 bytes, slot s of
// row r at s ^ ((r >> 1) & 3), so the 8 lanes of each read phase hit 8
// distinct 16-byte bank groups.  Rows past n0 and tokens past n1 read a clamped valid
// index: they feed only outputs that are never stored.
// ---------------------------------------------------------------------------
struct MxGemmArgs {
    const uint8_t* codes_w;    // [n0, K / 2]
    const uint8_t* scales_w;   // [n0, K / 32]
    const uint8_t* codes_a;    // [n1, K / 2]
    const uint8_t* scales_a;   // [n1, K / 32]
    float* z;                  // [n0, n1]
    int32_t n0, n1, K;
    int32_t tiles_j, tiles_n, per_xcd;
    uint32_t tiles;            // tiles_j * tiles_n (checked on the host)
};

typedef int v8i __attribute__((ext_vector_type(8)));

// One thread's share of a k step: 2 + TN / 64 code words and up to two
// scale words (weights row t for t < 128, activations row t for t < TN).
template <int TN, int TM>
struct MxStage {
    u4v w[TM / 64], x[TN / 64];
    uint32_t sw, sx;
};

// TN = 128 or 256 tokens per tile; each wave computes 64 weight rows x TN / 2
// tokens, so the wider tile reads 12 KB of LDS per 32 MFMAs instead of 8 KB
// per 16 (it pays from about a thousand tokens on).
template <int TN, int TM>
__global__ __launch_bounds__(kThreads) void k_mx_gemm(MxGemmArgs a) {
    // TM / 64 waves along the weight rows, the other 4 / (TM / 64) along the tokens
    constexpr int WM = TM / 64, WT = 4 / WM, NX = TN / 64, NB = TN / (16 * WT);
    __shared__ u4v sW[2][TM * 4], sA[2][TN * 4];          // codes, 64 bytes per row
    __shared__ uint32_t sWs[2][TM], sAs[2][TN];           // scale words, 4 E8M0 bytes per row
    const uint32_t b = blockIdx.x;
    const uint32_t idx = (b & 7u) * (uint32_t)a.per_xcd + (b >> 3);
    if (idx >= a.tiles) return;
    int jb, nb;
    gemm_tile_of<8>(idx, (uint32_t)a.tiles_j, (uint32_t)a.tiles_n, jb, nb);
    const int j0 = jb * TM, t0 = nb * TN;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WT, wn = wave % WT;
    const int nks = a.K / 128;
    const int64_t cstride = a.K / 2, sstride = a.K / 32;
    // staging: thread t moves 16-byte slot t & 3 of weight rows t / 4 + 64 i
    // (i < 2) and activation rows t / 4 + 64 i (i < 4), and the scale words
    // of weight row t (t < 128) and activation row t
    const int r0 = t >> 2, slot = t & 3;
    const uint8_t* gw[WM];
    const uint8_t* gx[NX];
    int lw[WM], lx[NX];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
        const int row = r0 + 64 * i;
        gw[i] = a.codes_w + (int64_t)min(j0 + row, a.n0 - 1) * cstride + slot * 16;
        lw[i] = row * 4 + (slot ^ ((row >> 1) & 3));
    }
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int row = r0 + 64 * i;
        gx[i] = a.codes_a + (int64_t)min(t0 + row, a.n1 - 1) * cstride + slot * 16;
        lx[i] = row * 4 + (slot ^ ((row >> 1) & 3));
    }
    const uint8_t* gsw = a.scales_w + (int64_t)min(j0 + (t % TM), a.n0 - 1) * sstride;
    const uint8_t* gsx = a.scales_a + (int64_t)min(t0 + (t % TN), a.n1 - 1) * sstride;
    auto load_stage = [&](int ks, MxStage<TN, TM>& r) {
#pragma unroll
        for (int i = 0; i < WM; ++i) r.w[i] = *reinterpret_cast<const u4v*>(gw[i] + ks * 64);
#pragma unroll
        for (int i = 0; i < NX; ++i) r.x[i] = *reinterpret_cast<const u4v*>(gx[i] + ks * 64);
        if (t < TM) r.sw = *reinterpret_cast<const uint32_t*>(gsw + ks * 4);
        if (t < TN) r.sx = *reinterpret_cast<const uint32_t*>(gsx + ks * 4);
    };
    auto store_stage = [&](const MxStage<TN, TM>& r, int buf) {
#pragma unroll
        for (int i = 0; i < WM; ++i) sW[buf][lw[i]] = r.w[i];
#pragma unroll
        for (int i = 0; i < NX; ++i) sA[buf][lx[i]] = r.x[i];
        if (t < TM) sWs[buf][t] = r.sw;
        if (t < TN) sAs[buf][t] = r.sx;
    };
    const int kb = lane >> 4;                 // this lane's 32-k block of a step
    f4v acc[4][NB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) acc[mt][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    MxStage<TN, TM> ra = {}, rb = {};
    load_stage(0, ra);
    if (nks > 1) load_stage(1, rb);
    store_stage(ra, 0);
    // registers: rb holds step ks + 1, then receives step ks + 2
    for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        lds_barrier();                        // step ks is in LDS; step ks - 1's buffer is free
        v8i af[4], bf[NB];
        int sa[4], sb[NB];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = wm * 64 + m * 16 + (lane & 15);
            const u4v c = sW[buf][r * 4 + (kb ^ ((r >> 1) & 3))];
            af[m] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
            sa[m] = (int)((sWs[buf][r] >> (8 * kb)) & 0xFFu);
        }
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const int r = wn * (TN / WT) + m * 16 + (lane & 15);
            const u4v c = sA[buf][r * 4 + (kb ^ ((r >> 1) & 3))];
            bf[m] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
            sb[m] = (int)((sAs[buf][r] >> (8 * kb)) & 0xFFu);
        }
        if (ks + 1 < nks) store_stage(rb, buf ^ 1);
        if (ks + 2 < nks) load_stage(ks + 2, rb);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NB; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mt], bf[nt], acc[mt][nt], 4, 4, 0,
                                                                               sa[mt], 0, sb[nt]);
    }
    // Non-temporal output stores: z passes through L2 without displacing the
    // operand tiles that neighbouring workgroups share (14336 x 4096 weights:
    // 114.3 -> 112.2 us at 2048 tokens, 405 -> 401 us at 8192, and a little
    // faster at 128 and 256; the BF16-activation consumers measured slower
    // this way at 2048 tokens and keep plain stores).
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + wm * 64 + mt * 16 + 4 * (lane >> 4) + i;
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int tok = t0 + wn * (TN / WT) + nt * 16 + (lane & 15);
                if (j < a.n0 && tok < a.n1) __builtin_nontemporal_store(acc[mt][nt][i], a.z + (int64_t)j * a.n1 + tok);
            }
        }
}

// Large products with the operand copies done by LDS DMA
// (global_load_lds): 256 x 256 tiles of 8 waves, 64 weight rows x 128
// tokens each (two waves per SIMD).  A stage is a pair of k steps, 128 code
// bytes per row: each 8 lanes of a DMA instruction fetch one row's whole
// 128-byte line, where the register-staged kernel fetched half lines (64
// bytes per row and step), which cost four L2 requests per 128 bytes against
// one.  No registers hold the copies.  The LDS row is 8 slots of 16 bytes,
// logical slot ls (step ls / 4, k block ls % 4) at ls ^ (r & 7); a lane's
// DMA word goes to a fixed LDS slot, so each lane fetches the logical slot
// that belongs there.  Scale words: 2 per row and pair (8 E8M0 bytes), read
// back as single bytes.  Two LDS stages (68 KB each): the copy of pair p + 1
// is issued after the barrier that opens pair p and lands during its MFMAs.
// With an odd step count the last pair's second step repeats the last step
// (in-bounds) and is not computed.  The two stages are separate LDS objects
// and the pair loop is unrolled by two, so that every read and every copy
// names its stage statically: with one array indexed by the stage the
// compiler waited for the next pair's copies before each LDS read
// (vmcnt(0)), which serialized copy and compute (c3 weights at 2048 / 8192
// tokens: 101.5 / 387 us that way, 94.3 / 348 us this way).
struct MxPairBuf {
    u4v w[256 * 8], a[256 * 8];
    uint32_t sw[256 * 2], sa[256 * 2];
};
__global__ __launch_bounds__(512) void k_mx_gemm_dma(MxGemmArgs a) {
    constexpr int TM = 256, TN = 256, WT = 2, NB = 8;
    __shared__ MxPairBuf P0, P1;
    const uint32_t b = blockIdx.x;
    const uint32_t idx = (b & 7u) * (uint32_t)a.per_xcd + (b >> 3);
    if (idx >= a.tiles) return;
    int jb, nb;
    gemm_tile_of<8>(idx, (uint32_t)a.tiles_j, (uint32_t)a.tiles_n, jb, nb);
    const int j0 = jb * TM, t0 = nb * TN;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WT, wn = wave % WT;
    const int nks = a.K / 128, np = (nks + 1) / 2;
    const int64_t cstride = a.K / 2, sstride = a.K / 32;
    // DMA lanes: instruction i of this wave covers rows 8 (4 wave + i) ..
    // + 7 of each operand; lane l takes row + (l >> 3), LDS slot l & 7,
    // which holds logical slot ls = (l & 7) ^ ((l >> 3) & 7)
    const int ls = (lane & 7) ^ ((lane >> 3) & 7), lhalf = ls >> 2, lkb = (ls & 3) * 16;
    const uint8_t* gw[4];
    const uint8_t* gx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + (lane >> 3);
        gw[i] = a.codes_w + (int64_t)min(j0 + row, a.n0 - 1) * cstride + lkb;
        gx[i] = a.codes_a + (int64_t)min(t0 + row, a.n1 - 1) * cstride + lkb;
    }
    // scale lanes: row 32 wave + (l >> 1), word l & 1 of the pair
    const int srow = 32 * wave + (lane >> 1), sword = lane & 1;
    const uint8_t* gsw = a.scales_w + (int64_t)min(j0 + srow, a.n0 - 1) * sstride;
    const uint8_t* gsx = a.scales_a + (int64_t)min(t0 + srow, a.n1 - 1) * sstride;
    auto issue = [&](int p, MxPairBuf& d) {
        const int64_t off = (int64_t)min(2 * p + lhalf, nks - 1) * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(gw[i] + off, (lds_void*)&d.w[(4 * wave + i) * 64], 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(gx[i] + off, (lds_void*)&d.a[(4 * wave + i) * 64], 16, 0, 0);
        const int64_t soff = (int64_t)min(2 * p + sword, nks - 1) * 4;
        __builtin_amdgcn_global_load_lds(gsw + soff, (lds_void*)&d.sw[wave * 64], 4, 0, 0);
        __builtin_amdgcn_global_load_lds(gsx + soff, (lds_void*)&d.sa[wave * 64], 4, 0, 0);
    };
    const int kb = lane >> 4;
    f4v acc[4][NB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) acc[mt][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    auto pair = [&](int p, const MxPairBuf& cur, MxPairBuf& nxt) {
        wait_staged();                        // this wave's copies of pair p have landed
        lds_barrier();                        // every wave's have; pair p - 1's tile is free
        if (p + 1 < np) issue(p + 1, nxt);
        const uint8_t* bw = reinterpret_cast<const uint8_t*>(cur.sw);
        const uint8_t* ba = reinterpret_cast<const uint8_t*>(cur.sa);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s == 1 && 2 * p + 1 >= nks) break;   // uniform: odd step count
            const int lsl = 4 * s + kb;
            v8i af[4], bf[NB];
            int sa[4], sb[NB];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = wm * 64 + m * 16 + (lane & 15);
                const u4v c = cur.w[r * 8 + (lsl ^ (r & 7))];
                af[m] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
                sa[m] = bw[r * 8 + lsl];
            }
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const int r = wn * 128 + m * 16 + (lane & 15);
                const u4v c = cur.a[r * 8 + (lsl ^ (r & 7))];
                bf[m] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
                sb[m] = ba[r * 8 + lsl];
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mt], bf[nt], acc[mt][nt], 4, 4, 0,
                                                                                   sa[mt], 0, sb[nt]);
        }
    };
    issue(0, P0);
    for (int p = 0; p < np; p += 2) {
        pair(p, P0, P1);
        if (p + 1 < np) pair(p + 1, P1, P0);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + wm * 64 + mt * 16 + 4 * (lane >> 4) + i;
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int tok = t0 + wn * 128 + nt * 16 + (lane & 15);
                if (j < a.n0 && tok < a.n1) __builtin_nontemporal_store(acc[mt][nt][i], a.z + (int64_t)j * a.n1 + tok);
            }
        }
}

// Few tokens (n1 <= 64) for the FP4 GEMM: the weights stream once, so HBM
// bounds the call.  A workgroup takes 32 weight rows and 16 NT tokens (16
// rows per workgroup measured slower from 16 tokens on); its 4 waves split the
// pairs of k steps (wave w takes pairs w, w + 4, ...) and load the MFMA
// operands straight from memory into registers (no LDS tile); the waves'
// partial sums meet in LDS at the end, added in wave order.  The
// activations are operand A (rows = tokens) and the weights operand B
// (columns = weight rows): lane l loads weight row 16 f + l % 16 and
// receives results of that row for tokens 4 (l / 16) .. + 3.
// Rows past n0 and tokens past n1 read a clamped valid index; a pair past
// the last step (odd step count) reads nothing beyond a row.
template <int NT>
struct MxGemvPair {
    u4v c[2][2];          // weight codes [fragment][step of the pair]
    u4v x[2][NT];         // activation codes [step][token tile]
};

constexpr int kMxGemvChunk = 32;   // pairs of steps whose scale words one LDS chunk holds

// The scale words (4 E8M0 bytes per row and step) of the workgroup's 32
// weight rows and 16 NT tokens reach LDS in chunks, with coalesced loads:
// read per lane, 16 rows apart, they cost about a fifth of the call.
template <int NT>
__global__ __launch_bounds__(kThreads) void k_mx_gemv(MxGemmArgs a) {
    __shared__ f4v red[4][2][NT][64];
    __shared__ uint32_t s_sw[32][2 * kMxGemvChunk + 1];
    __shared__ uint32_t s_sx[16 * NT][2 * kMxGemvChunk + 1];
    const int j0 = (int)blockIdx.x * 32, t0 = (int)blockIdx.y * 16 * NT;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int rr = lane & 15, h = lane >> 4;
    const int nks = a.K / 128, np = (nks + 1) / 2;
    const int64_t cstride = a.K / 2, sstride = a.K / 32;
    const uint8_t* cw[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int64_t j = min(j0 + 16 * f + rr, a.n0 - 1);
        cw[f] = a.codes_w + j * cstride + 16 * h;
    }
    const uint8_t* cx[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t tok = min(t0 + 16 * nt + rr, a.n1 - 1);
        cx[nt] = a.codes_a + tok * cstride + 16 * h;
    }
    auto load_pair = [&](int p, MxGemvPair<NT>& w) {
        const bool both = 2 * p + 1 < nks;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (e == 1 && !both) break;
#pragma unroll
            for (int f = 0; f < 2; ++f) w.c[f][e] = *reinterpret_cast<const u4v*>(cw[f] + p * 128 + e * 64);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) w.x[e][nt] = *reinterpret_cast<const u4v*>(cx[nt] + p * 128 + e * 64);
        }
    };
    f4v acc[2][NT];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[f][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    // pc: the pair's index within the staged chunk
    auto compute_pair = [&](int p, int pc, const MxGemvPair<NT>& w) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int ks = 2 * p + e;
            if (ks >= nks) break;
            v8i xa[NT];
            int xs[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const u4v c = w.x[e][nt];
                xa[nt] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
                xs[nt] = (int)((s_sx[16 * nt + rr][2 * pc + e] >> (8 * h)) & 0xFFu);
            }
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const u4v c = w.c[f][e];
                const v8i wb = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
                const int ws = (int)((s_sw[16 * f + rr][2 * pc + e] >> (8 * h)) & 0xFFu);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[f][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa[nt], wb, acc[f][nt], 4, 4, 0,
                                                                                   xs[nt], 0, ws);
            }
        }
    };
    // The wave's pairs in chunks of kMxChunk, every load of a chunk issued
    // before any of its math: enough bytes in flight per CU to stream the
    // weights at HBM rate when each wave owns only a few pairs.
    constexpr int kMxChunk = NT == 4 ? 2 : 4;
    for (int c0 = 0; c0 < np; c0 += kMxGemvChunk) {
        const int c1 = min(np, c0 + kMxGemvChunk);
        const int cs = min(2 * c1, nks) - 2 * c0;   // steps in the staged chunk
        __syncthreads();                            // the previous chunk's scales are no longer read
        for (int i = t; i < 32 * cs; i += kThreads) {
            const int r = i / cs, ss = i - r * cs;
            s_sw[r][ss] = *reinterpret_cast<const uint32_t*>(a.scales_w + min(j0 + r, a.n0 - 1) * sstride +
                                                              4 * (2 * c0 + ss));
        }
        for (int i = t; i < 16 * NT * cs; i += kThreads) {
            const int r = i / cs, ss = i - r * cs;
            s_sx[r][ss] = *reinterpret_cast<const uint32_t*>(a.scales_a + min(t0 + r, a.n1 - 1) * sstride +
                                                              4 * (2 * c0 + ss));
        }
        __syncthreads();
        for (int p0 = c0 + wave; p0 < c1; p0 += 4 * kMxChunk) {
            MxGemvPair<NT> pr[kMxChunk];
#pragma unroll
            for (int c = 0; c < kMxChunk; ++c) load_pair(min(p0 + 4 * c, c1 - 1), pr[c]);
#pragma unroll
            for (int c = 0; c < kMxChunk; ++c)
                if (p0 + 4 * c < c1) compute_pair(p0 + 4 * c, p0 + 4 * c - c0, pr[c]);
        }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave][f][nt][lane] = acc[f][nt];
    __syncthreads();
    const int part = t >> 6;
#pragma unroll
    for (int fi = 0; fi < 2 * NT; ++fi) {
        if (fi % 4 != part) continue;
        const int f = fi / NT, nt = fi % NT;
        const int j = j0 + 16 * f + rr;
        if (j >= a.n0) continue;
        const f4v v = ((red[0][f][nt][lane] + red[1][f][nt][lane]) + red[2][f][nt][lane]) + red[3][f][nt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * nt + 4 * h + i;
            if (tok < a.n1) a.z[(int64_t)j * a.n1 + tok] = v[i];
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4 weights against BF16 activations (W4A16):
//   z[j, t] = sum_k xw[j, k] * x[t, k],  xw = 2^(E - 127) * e2m1(code)
// (low-precision post, "FP4 / MXFP4 / NVFP4").  A 16-byte code word is one
// block of 32 (one E8M0 scale); v_cvt_scalef32_pk_bf16_fp4 turns two codes
// into two BF16 weights scaled by the block's power of two, exactly (an
// E2M1 value times a power of two has at most 2 significant bits).  The BF16
// matrix cores then form exact products with the activations and sum in
// FP32: no per-block fold, and 0.5 VALU instructions per weight.  E8M0 255
// (NaN) gives NaN weights.  The kernels are the asymmetric INT4 consumer's
// (LDS tiles from 65 tokens, registers only below) with this
// dequantization; where the INT4 kernel splits k for small grids, these
// take 64-row tiles (TM = 64, 1 x 4 waves of 64 x 32).
// ---------------------------------------------------------------------------
struct MxwGemmArgs {
    const uint8_t* codes;      // [n0, K / 2]
    const uint8_t* scales;     // [n0, K / 32] E8M0
    const uint16_t* x;         // [n1, K] BF16
    float* z;                  // [n0, n1]
    int32_t n0, n1, K;
    int32_t tiles_j, tiles_n, per_xcd;
    uint32_t tiles;            // tiles_j * tiles_n (checked on the host)
};

// 8 weights of one code word (element 2t in the low nibble of byte t) as
// BF16 times the block scale sc (a power of two; NaN for E8M0 255).
__device__ __forceinline__ u4v mx_bf16x8(uint32_t w, float sc, bool nan) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    u4v o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    if (nan) o = u4v{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    return o;
}
__device__ __forceinline__ float e8m0_scale(uint32_t E) {
    return E ? as_f(E << 23) : as_f(0x00400000u);   // 2^(E - 127); 2^-127 is an FP32 subnormal
}

template <int WN, int TM>
__global__ __launch_bounds__(128 * WN) void k_mxw_gemm(MxwGemmArgs a) {
    constexpr int kTN = 64 * WN;             // tokens per tile
    constexpr int WR = TM / 64, WT = 2 * WN / WR;   // waves along rows and along tokens
    constexpr int NB = kTN / WT / 16;        // 16-token MFMA blocks per wave
    constexpr int TPR = 128 * WN / TM;       // staging threads per weight row
    constexpr int kWords = 4 / TPR;          // 16-byte code words (scale blocks) per thread and step
    constexpr int kX = 8;                    // 16-byte activation words per thread and step
    __shared__ u4v tiles[(TM + kTN) * 16];
    u4v* const sA = tiles;                   // weights BF16, swizzled rows of 128
    u4v* const sB = tiles + TM * 16;         // activations BF16, same layout
    const uint32_t b = blockIdx.x;
    const uint32_t idx = (b & 7u) * (uint32_t)a.per_xcd + (b >> 3);
    if (idx >= a.tiles) return;
    int jb, nb;
    gemm_tile_of<16>(idx, (uint32_t)a.tiles_j, (uint32_t)a.tiles_n, jb, nb);
    const int j0 = jb * TM, t0 = nb * kTN;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WT, wn = wave % WT;
    const int nks = a.K / 128;
    const int ldc = a.K / 2, lds_ = a.K / 32;
    f4v acc[4][NB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) acc[mt][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    // staging: thread t moves 16-byte slot t & 15 of token rows t / 16 + 8 WN i
    // (i < 8), and the code words of weight row t / WN (blocks dp * kWords ..)
    const int xr0 = t >> 4, xs = t & 15;
    const uint16_t* gx[kX];
    int lx[kX];
#pragma unroll
    for (int i = 0; i < kX; ++i) {
        const int row = xr0 + 8 * WN * i;
        gx[i] = a.x + (int64_t)min(t0 + row, a.n1 - 1) * a.K + xs * 8;
        lx[i] = row * 16 + (xs ^ (row & 15));
    }
    const int dr = t / TPR, dp = t % TPR;
    const int64_t dj = min(j0 + dr, a.n0 - 1);
    const u4v* gc = reinterpret_cast<const u4v*>(a.codes + dj * ldc + dp * 16 * kWords);
    const uint8_t* gs = a.scales + dj * lds_ + dp * kWords;
    u4v rx[kX], rc[kWords];
    uint32_t rs[kWords];
    auto load_step = [&](int ks) {
#pragma unroll
        for (int i = 0; i < kX; ++i) rx[i] = *reinterpret_cast<const u4v*>(gx[i] + ks * 128);
#pragma unroll
        for (int v = 0; v < kWords; ++v) {
            rc[v] = gc[ks * 4 + v];
            rs[v] = gs[ks * 4 + v];
        }
    };
    load_step(0);
    for (int ks = 0; ks < nks; ++ks) {
        __syncthreads();                     // every wave is done with the previous step's tiles
#pragma unroll
        for (int i = 0; i < kX; ++i) sB[lx[i]] = rx[i];
#pragma unroll
        for (int v = 0; v < kWords; ++v) {
            const float sc = e8m0_scale(rs[v]);
            const uint32_t cw[4] = {rc[v].x, rc[v].y, rc[v].z, rc[v].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sA[dr * 16 + ((dp * 4 * kWords + 4 * v + q) ^ (dr & 15))] = mx_bf16x8(cw[q], sc, rs[v] == 255u);
        }
        if (ks + 1 < nks) load_step(ks + 1);     // lands during this step's MFMAs
        lds_barrier();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int slot = 4 * s + (lane >> 4);
            bf8v af[4], bfr[NB];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int r = wm * 64 + mt * 16 + (lane & 15);
                af[mt] = __builtin_bit_cast(bf8v, sA[r * 16 + (slot ^ (r & 15))]);
            }
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int r = wn * (kTN / WT) + nt * 16 + (lane & 15);
                bfr[nt] = __builtin_bit_cast(bf8v, sB[r * 16 + (slot ^ (r & 15))]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + wm * 64 + mt * 16 + 4 * (lane >> 4) + i;
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int tok = t0 + wn * (kTN / WT) + nt * 16 + (lane & 15);
                if (j < a.n0 && tok < a.n1) a.z[(int64_t)j * a.n1 + tok] = acc[mt][nt][i];
            }
        }
}

// Large grids: 256 x 256 tiles, 8 waves of 64 weight rows x 128 tokens (two
// waves per SIMD), double-buffered in k steps of 64.  A step reads 0.375 KB
// of LDS fragments per MFMA against 0.5 for the 64 x 64 wave tiles above,
// and with the LDS writes the tile's LDS time per step falls to about its
// MFMA time.  Rows of a step are 128 bytes (8 slots of 16, slot s of row r at
// s ^ (r & 7)); two tiles of 64 KB.  Step k + 1 is written to the other tile
// while step k's MFMAs run, and step k + 2 loads into registers; one
// LDS-only barrier per step.  Every thread also dequantizes one 32-code
// block per step (weight row t / 2, block t % 2).  Measured on the c3
// weights (14336 x 4096) against the 128 x 256 tiles: 141 -> 112 us at 1024
// tokens, 279 -> 224 us at 2048, 967 -> 836 us at 8192; the 128 x 256 tile
// double-buffered the same way gained 0-2.5%.
__global__ __launch_bounds__(512) void k_mxw_gemm_wide(MxwGemmArgs a) {
    constexpr int kTN = 256, TM = 256, WT = 2, NB = 8;
    __shared__ u4v sA[2][TM * 8], sB[2][kTN * 8];
    const uint32_t b = blockIdx.x;
    const uint32_t idx = (b & 7u) * (uint32_t)a.per_xcd + (b >> 3);
    if (idx >= a.tiles) return;
    int jb, nb;
    gemm_tile_of<16>(idx, (uint32_t)a.tiles_j, (uint32_t)a.tiles_n, jb, nb);
    const int j0 = jb * TM, t0 = nb * kTN;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WT, wn = wave % WT;
    const int nks = a.K / 64;
    const int ldc = a.K / 2, lds_ = a.K / 32;
    f4v acc[4][NB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) acc[mt][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    const int xr0 = t >> 3, xs = t & 7;
    const uint16_t* gx[4];
    int lx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = xr0 + 64 * i;
        gx[i] = a.x + (int64_t)min(t0 + row, a.n1 - 1) * a.K + xs * 8;
        lx[i] = row * 8 + (xs ^ (row & 7));
    }
    const int dr = t >> 1, dp = t & 1;
    const int64_t dj = min(j0 + dr, a.n0 - 1);
    const u4v* gc = reinterpret_cast<const u4v*>(a.codes + dj * ldc + dp * 16);
    const uint8_t* gs = a.scales + dj * lds_ + dp;
    u4v rx[4], rc = {};
    uint32_t rs = 0;
    auto load_step = [&](int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rx[i] = *reinterpret_cast<const u4v*>(gx[i] + ks * 64);
        rc = gc[ks * 2];
        rs = gs[ks * 2];
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sB[buf][lx[i]] = rx[i];
        const float sc = e8m0_scale(rs);
        const uint32_t cw[4] = {rc.x, rc.y, rc.z, rc.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) sA[buf][dr * 8 + ((dp * 4 + q) ^ (dr & 7))] = mx_bf16x8(cw[q], sc, rs == 255u);
    };
    load_step(0);
    store_step(0);
    if (nks > 1) load_step(1);
    for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        lds_barrier();                        // step ks is in LDS; step ks - 1's tile is free
        if (ks + 1 < nks) store_step(buf ^ 1);
        if (ks + 2 < nks) load_step(ks + 2);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int slot = 4 * s + (lane >> 4);
            bf8v af[4], bfr[NB];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int r = wm * 64 + mt * 16 + (lane & 15);
                af[mt] = __builtin_bit_cast(bf8v, sA[buf][r * 8 + (slot ^ (r & 7))]);
            }
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int r = wn * (kTN / WT) + nt * 16 + (lane & 15);
                bfr[nt] = __builtin_bit_cast(bf8v, sB[buf][r * 8 + (slot ^ (r & 7))]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + wm * 64 + mt * 16 + 4 * (lane >> 4) + i;
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int tok = t0 + wn * (kTN / WT) + nt * 16 + (lane & 15);
                if (j < a.n0 && tok < a.n1) a.z[(int64_t)j * a.n1 + tok] = acc[mt][nt][i];
            }
        }
}

// Few tokens (n1 <= 64): the asymmetric INT4 consumer's register-only kernel
// with this dequantization.  Lane l holds weight row 16 f + l % 16 and, for
// MFMA step q of 128-deep step g, k = 128 g + 32 (l / 16) + 8 q .. + 8: one
// word of its 16-byte code load, whose block scale is byte 4 g + l / 16 of
// the row.  A step past the last one (odd step count) reads nothing.
template <int FR> struct MxwPair {
    u4v c[FR][2];          // codes [fragment][step of the pair]
};

// Scale words (4 E8M0 bytes per row and step) reach LDS in chunks of up to
// kGemvChunk pairs of steps, as for the asymmetric INT4 kernel; so do the
// load order (a pair's activations before the next pair's codes), the
// stripes of 16 FR rows (FR = 4 from 9 to 32 tokens) and, with X1 (a single
// token), the activation row's slice.
template <int NT, bool X1, int FR>
__global__ __launch_bounds__(kThreads, NT == 1 ? (FR == 2 ? 4 : 3) : 1) void k_mxw_gemv(MxwGemmArgs a) {
    constexpr int kRows = 16 * FR;
    static_assert(!X1 || NT == 1, "one token, one token tile");
    __shared__ f4v red[4][FR][NT][64];
    __shared__ uint32_t s_sw[kRows][2 * kGemvChunk + 1];
    __shared__ u4v s_x[X1 ? 2 * kGemvChunk * 16 : 1];
    const int j0 = (int)blockIdx.x * kRows, t0 = (int)blockIdx.y * 16 * NT;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int rr = lane & 15, h = lane >> 4;
    const int nks = a.K / 128, np = (nks + 1) / 2;
    const uint8_t* crow[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
        const int64_t j = min(j0 + 16 * f + rr, a.n0 - 1);
        crow[f] = a.codes + j * (a.K / 2) + 16 * h;
    }
    const u4v* xr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t tok = min(t0 + 16 * nt + rr, a.n1 - 1);
        xr[nt] = reinterpret_cast<const u4v*>(a.x + tok * a.K + 32 * h);
    }
    auto load_pair = [&](int p, MxwPair<FR>& w) {
        const bool both = 2 * p + 1 < nks;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (e == 1 && !both) break;
#pragma unroll
            for (int f = 0; f < FR; ++f) w.c[f][e] = *reinterpret_cast<const u4v*>(crow[f] + p * 128 + e * 64);
        }
    };
    auto load_x = [&](int p, int pc, u4v (&xw)[2][NT][4]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (2 * p + e >= nks) break;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xw[e][nt][q] = X1 ? s_x[(2 * pc + e) * 16 + 4 * h + q] : xr[nt][(2 * p + e) * 16 + q];
        }
    };
    f4v acc[FR][NT];
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[f][nt] = f4v{0.f, 0.f, 0.f, 0.f};
    // pc: the pair's index within the staged chunk
    auto compute_pair = [&](int p, int pc, const MxwPair<FR>& w, const u4v (&xp)[2][NT][4]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (2 * p + e >= nks) break;
#pragma unroll
            for (int f = 0; f < FR; ++f) {
                const uint32_t E = (s_sw[16 * f + rr][2 * pc + e] >> (8 * h)) & 0xFFu;
                const float sc = e8m0_scale(E);
                const uint32_t cw[4] = {w.c[f][e].x, w.c[f][e].y, w.c[f][e].z, w.c[f][e].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf8v bw = __builtin_bit_cast(bf8v, mx_bf16x8(cw[q], sc, E == 255u));
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[f][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, xp[e][nt][q]), bw,
                                                                              acc[f][nt], 0, 0, 0);
                }
            }
        }
    };
    for (int p0 = 0; p0 < np; p0 += kGemvChunk) {
        const int p1 = min(np, p0 + kGemvChunk);
        const int cs = min(2 * p1, nks) - 2 * p0;   // steps in the chunk
        __syncthreads();                            // the previous chunk's scales are no longer read
        for (int i = t; i < kRows * cs; i += kThreads) {
            const int r = i / cs, ss = i - r * cs;
            s_sw[r][ss] = *reinterpret_cast<const uint32_t*>(a.scales + (int64_t)min(j0 + r, a.n0 - 1) * (a.K / 32) +
                                                              4 * (2 * p0 + ss));
        }
        if (X1) {
            const u4v* xg = reinterpret_cast<const u4v*>(a.x) + (int64_t)(2 * p0) * 16;
            for (int i = t; i < cs * 16; i += kThreads) s_x[i] = xg[i];
        }
        __syncthreads();
        if (p0 + wave < p1) {
            MxwPair<FR> pa = {}, pb = {};
            u4v xw[2][NT][4] = {};
            load_pair(p0 + wave, pa);
            for (int p = p0 + wave; p < p1; p += 8) {
                load_x(p, p - p0, xw);
                asm volatile("" ::: "memory");
                load_pair(min(p + 4, p1 - 1), pb);
                compute_pair(p, p - p0, pa, xw);
                load_x(min(p + 4, p1 - 1), min(p + 4, p1 - 1) - p0, xw);
                asm volatile("" ::: "memory");
                load_pair(min(p + 8, p1 - 1), pa);
                if (p + 4 < p1) compute_pair(p + 4, p + 4 - p0, pb, xw);
            }
        }
    }
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave][f][nt][lane] = acc[f][nt];
    __syncthreads();
    const int part = t >> 6;
#pragma unroll
    for (int fi = 0; fi < FR * NT; ++fi) {
        if (fi % 4 != part) continue;
        const int f = fi / NT, nt = fi % NT;
        const int j = j0 + 16 * f + rr;
        if (j >= a.n0) continue;
        const f4v v = ((red[0][f][nt][lane] + red[1][f][nt][lane]) + red[2][f][nt][lane]) + red[3][f][nt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * nt + 4 * h + i;
            if (tok < a.n1) a.z[(int64_t)j * a.n1 + tok] = v[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side helpers.
// ---------------------------------------------------------------------------
int ilog2_exact(uint32_t v) {
    if (v == 0 || (v & (v - 1))) return -1;
    int s = 0;
    while ((1u << s) != v) ++s;
    return s;
}

FlatGeom make_geom(const void* x, int64_t rows, int64_t cols, int64_t ld) {
    FlatGeom g;
    g.x = x;
    g.ld = ld;
    g.cpr = (uint32_t)(cols / kChunk);
    g.nchunks = (uint32_t)(rows * (cols / kChunk));
    g.cpr_shift = ilog2_exact(g.cpr);
    g.contiguous = ld == cols;
    return g;
}

// Workgroups that fit on the device at once for a kernel (occupancy x CUs),
// capped by the partial slots of the workspace.  Persistent kernels launch
// at most this many, so no workgroup waits for a second wave of residency.
// Cached per (kernel, device); the cache is shared by host threads.
int resident_slots(const void* kernel, int threads) {
    static std::mutex mu;
    static std::unordered_map<uint64_t, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return kMaxGrid;
    const uint64_t key = reinterpret_cast<uint64_t>(kernel) * 64u + (uint64_t)dev;
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess || per <= 0) per = 1;
    int slots = per * cus;
    if (slots > kMaxGrid) slots = kMaxGrid;
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = slots;
    return slots;
}

template <int NT = kThreads, typename K> int grid_for(K kernel, uint64_t units) {
    const int slots = resident_slots(reinterpret_cast<const void*>(kernel), NT);
    if (units == 0) return 1;
    return units < (uint64_t)slots ? (int)units : slots;
}

// Per-row kernels take at least kRowsPerGroup rows per workgroup.  The last
// round of rows is cast after the final loads have landed, with nothing left
// to overlap it; a grid of half the resident slots halves that drain while
// still keeping enough loads in flight (BF16 8192 x 8192 E4M3 with
// statistics: 46.1 -> 44.1 us at 8 rows per workgroup, 48.4 at 6, 47.0 at
// 16; without statistics unchanged).
constexpr uint64_t kRowsPerGroup = 8;
template <int NT, typename K> int grid_for_rows(K kernel, uint64_t rows) {
    return grid_for<NT>(kernel, (rows + kRowsPerGroup - 1) / kRowsPerGroup);
}

uint32_t tiles_of(uint32_t nchunks) { return (nchunks + kTileChunks - 1) / kTileChunks; }

// With x^ requested the partial-row instantiation with statistics serves
// every row length (without a statistics output its partials go unread).
template <int IN, int FMT, int CPT, int NT, bool STATS>
void launch_row_k(const RowArgs& r, int& grid, hipStream_t s) {
    if (r.xhat) {
        grid = grid_for_rows<NT>(k_quant_row<IN, FMT, CPT, NT, false, true, true>, (uint64_t)r.rows);
        k_quant_row<IN, FMT, CPT, NT, false, true, true><<<grid, NT, 0, s>>>(r);
    } else if (r.cpr == CPT * NT) {
        grid = grid_for_rows<NT>(k_quant_row<IN, FMT, CPT, NT, true, false, STATS>, (uint64_t)r.rows);
        k_quant_row<IN, FMT, CPT, NT, true, false, STATS><<<grid, NT, 0, s>>>(r);
    } else {
        grid = grid_for_rows<NT>(k_quant_row<IN, FMT, CPT, NT, false, false, STATS>, (uint64_t)r.rows);
        k_quant_row<IN, FMT, CPT, NT, false, false, STATS><<<grid, NT, 0, s>>>(r);
    }
}

// Rows of up to 256 chunks take a one-wave workgroup (no cross-wave
// reduction); rows of up to 1024 chunks four waves, rows of up to 2048
// eight waves, with at most 4 chunks per lane; beyond that the two-pass
// kernel.  At 1024 chunks per row four waves with 4 chunks per lane measure
// faster than one wave with 16 (whose 200 VGPRs halve the resident waves),
// and at 2048 eight waves with 4 faster than four with 8 (about 200 VGPRs,
// 2 waves per SIMD against 8).
template <int IN, int FMT, bool STATS>
hipError_t launch_row_t(const RowArgs& r, int& grid, hipStream_t s) {
    const int cpr = r.cpr;
    if (cpr <= 64) launch_row_k<IN, FMT, 1, 64, STATS>(r, grid, s);
    else if (cpr <= 128) launch_row_k<IN, FMT, 2, 64, STATS>(r, grid, s);
    else if (cpr <= 256) launch_row_k<IN, FMT, 4, 64, STATS>(r, grid, s);
    else if (cpr <= 512) launch_row_k<IN, FMT, 2, kThreads, STATS>(r, grid, s);
    else if (cpr <= 1024) launch_row_k<IN, FMT, 4, kThreads, STATS>(r, grid, s);
    else if (cpr <= 2048) launch_row_k<IN, FMT, 4, 512, STATS>(r, grid, s);   // 8 waves per row
    else {
        grid = grid_for(k_quant_row_long<IN, FMT, STATS>, (uint64_t)r.rows);
        k_quant_row_long<IN, FMT, STATS><<<grid, kThreads, 0, s>>>(r);
    }
    return hipGetLastError();
}

template <int IN, int FMT>
hipError_t launch_row(const RowArgs& r, bool stats, int& grid, hipStream_t s) {
    return stats ? launch_row_t<IN, FMT, true>(r, grid, s) : launch_row_t<IN, FMT, false>(r, grid, s);
}

// Per-tensor INT8 / FP8 of a contiguous BF16 tensor whose size is a multiple
// of kTensorRowCols, as rows of that many elements under the tensor's
// scale: the per-row kernel's staging (two rows of 32 KB in flight per
// workgroup of eight waves, the waves kept on one row) moves the tensor
// faster than the flat kernel (BF16 65536 x 16384 INT8 per tensor, the
// whole call with its absmax pre-pass: 911 -> 875 us with statistics,
// 887 -> 858 us without).
constexpr int64_t kTensorRowCols = 16384;
template <int FMT, bool STATS>
hipError_t launch_row_tensor_k(const RowArgs& r, int& grid, hipStream_t s) {
    grid = grid_for_rows<512>(k_quant_row<D_BF16, FMT, 4, 512, true, false, STATS, true>, (uint64_t)r.rows);
    k_quant_row<D_BF16, FMT, 4, 512, true, false, STATS, true><<<grid, 512, 0, s>>>(r);
    return hipGetLastError();
}
hipError_t launch_row_tensor(int fmt, const RowArgs& r, bool stats, int& grid, hipStream_t s) {
    switch (fmt) {
    case F_INT8: return stats ? launch_row_tensor_k<F_INT8, true>(r, grid, s) : launch_row_tensor_k<F_INT8, false>(r, grid, s);
    case F_E4M3: return stats ? launch_row_tensor_k<F_E4M3, true>(r, grid, s) : launch_row_tensor_k<F_E4M3, false>(r, grid, s);
    default: return stats ? launch_row_tensor_k<F_E5M2, true>(r, grid, s) : launch_row_tensor_k<F_E5M2, false>(r, grid, s);
    }
}

template <int IN, int FMT, bool STATS, bool CHECK, bool XHAT>
hipError_t launch_flat_one(const FlatArgs& f, int& grid, hipStream_t s) {
    grid = grid_for(k_quant_flat<IN, FMT, STATS, CHECK, XHAT>, tiles_of(f.geo.nchunks));
    k_quant_flat<IN, FMT, STATS, CHECK, XHAT><<<grid, kThreads, 0, s>>>(f);
    return hipGetLastError();
}

// check: per-tensor INT8 / FP8 with a caller-supplied absmax (the other
// formats decide per block and need no data checks).  With x^ requested the
// instantiation with statistics serves (without a statistics output its
// partials go unread).
template <int IN, int FMT, bool CHECK>
hipError_t launch_flat_c(const FlatArgs& f, bool stats, int& grid, hipStream_t s) {
    if (f.xhat) return launch_flat_one<IN, FMT, true, CHECK, true>(f, grid, s);
    return stats ? launch_flat_one<IN, FMT, true, CHECK, false>(f, grid, s)
                 : launch_flat_one<IN, FMT, false, CHECK, false>(f, grid, s);
}

template <int IN, int FMT>
hipError_t launch_flat(const FlatArgs& f, bool stats, bool check, int& grid, hipStream_t s) {
    constexpr bool kUniform = FMT == F_INT8 || FMT == F_E4M3 || FMT == F_E5M2;
    if (kUniform && check) return launch_flat_c<IN, FMT, kUniform>(f, stats, grid, s);
    return launch_flat_c<IN, FMT, false>(f, stats, grid, s);
}

template <int IN>
hipError_t launch_flat_fmt(int fmt, const FlatArgs& f, bool stats, bool check, int& grid, hipStream_t s) {
    switch (fmt) {
    case F_INT8: return launch_flat<IN, F_INT8>(f, stats, check, grid, s);
    case F_E4M3: return launch_flat<IN, F_E4M3>(f, stats, check, grid, s);
    case F_E5M2: return launch_flat<IN, F_E5M2>(f, stats, check, grid, s);
    case F_MXFP4: return launch_flat<IN, F_MXFP4>(f, stats, check, grid, s);
    case F_NVFP4: return launch_flat<IN, F_NVFP4>(f, stats, check, grid, s);
    case F_INT4ZP: return launch_flat<IN, F_INT4ZP>(f, stats, check, grid, s);
    default: return launch_flat<IN, F_INT4>(f, stats, check, grid, s);
    }
}

template <int IN>
hipError_t launch_row_fmt(int fmt, const RowArgs& r, bool stats, int& grid, hipStream_t s) {
    switch (fmt) {
    case F_INT8: return launch_row<IN, F_INT8>(r, stats, grid, s);
    case F_E4M3: return launch_row<IN, F_E4M3>(r, stats, grid, s);
    default: return launch_row<IN, F_E5M2>(r, stats, grid, s);
    }
}

// The absmax pass in one launch.  fold: its last workgroup writes the
// results (an empty tensor takes one workgroup, which writes zeros);
// otherwise each workgroup leaves its word at Workspace::kAmaxOff for the
// cast kernel, and *grid_out is the number of words.
template <int IN>
void launch_amax_k(const FlatGeom& geo, const AmaxSink& k, bool fold, int& grid, hipStream_t s) {
    if (fold) {
        grid = grid_for(k_amax<IN, true>, tiles_of(geo.nchunks));
        k_amax<IN, true><<<grid, kThreads, 0, s>>>(geo, k);
    } else {
        grid = grid_for(k_amax<IN, false>, tiles_of(geo.nchunks));
        k_amax<IN, false><<<grid, kThreads, 0, s>>>(geo, k);
    }
}

hipError_t launch_amax_pass(int in_dtype, const FlatGeom& geo, void* ws, bool fold, float qdiv, float* scale_out,
                            float* amax_out, int* grid_out, hipStream_t s) {
    AmaxSink k;
    k.partials = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + Workspace::kAmaxOff);
    k.ticket = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + Workspace::kAmaxTicketOff);
    k.qdiv = qdiv; k.scale_out = scale_out; k.amax_out = amax_out;
    int grid = 0;
    if (in_dtype == D_BF16) launch_amax_k<D_BF16>(geo, k, fold, grid, s);
    else launch_amax_k<D_F32>(geo, k, fold, grid, s);
    if (grid_out) *grid_out = grid;
    return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_quantize(const QuantArgs& q, hipStream_t s) {
    char* ws = static_cast<char*>(q.workspace);
    const bool stats = q.stats != nullptr;
    const int64_t nelem = q.rows * q.cols;
    StatsSink sink;
    sink.partials = reinterpret_cast<Partial*>(ws + Workspace::kPartialOff);
    sink.ticket = reinterpret_cast<uint32_t*>(ws + Workspace::kStatsTicketOff);
    sink.out = static_cast<StatsOut*>(q.stats);
    sink.nelem = (uint64_t)nelem;
    int grid = 0;
    bool stats_written = false;   // a quantize kernel with statistics ran (its last workgroup wrote them)
    hipError_t e = hipSuccess;

    if (q.gran == G_ROW) {
        RowArgs r;
        r.x = q.x; r.ld = q.ld; r.rows = (int32_t)q.rows; r.cpr = (int32_t)(q.cols / kChunk);
        r.codes = static_cast<uint8_t*>(q.codes); r.scales = static_cast<float*>(q.scales);
        r.xhat = q.xhat; r.xhat_dtype = q.xhat_dtype; r.sink = sink;
        r.amax_words = nullptr; r.amax_nwords = 0; r.scale_out = nullptr;
        if (nelem) {
            e = q.in_dtype == D_BF16 ? launch_row_fmt<D_BF16>(q.fmt, r, stats, grid, s)
                                     : launch_row_fmt<D_F32>(q.fmt, r, stats, grid, s);
            stats_written = true;
        }
    } else {
        FlatArgs f;
        f.geo = make_geom(q.x, q.rows, q.cols, q.ld);
        f.codes = static_cast<uint8_t*>(q.codes); f.scales = q.scales; f.global_scale = q.global_scale;
        f.xhat = q.xhat; f.xhat_dtype = q.xhat_dtype; f.sink = sink;
        f.amax_words = reinterpret_cast<const uint64_t*>(ws + Workspace::kAmaxOff);
        f.amax_nwords = 0;
        f.rule = q.rule;
        f.shifts = q.shifts;
        f.static_amax = q.static_amax;
        f.scale_out = q.fmt == F_NVFP4 ? q.global_scale : static_cast<float*>(q.scales);
        if ((q.gran == G_TENSOR || q.fmt == F_NVFP4) && !q.static_amax) {
            // A non-empty tensor's cast kernel folds the pre-pass words itself;
            // an empty one has no cast kernel, so its pre-pass writes the scale.
            const float qdiv = q.fmt == F_INT8 ? 127.f : q.fmt == F_E4M3 ? 448.f : q.fmt == F_E5M2 ? 57344.f : 2688.f;
            e = launch_amax_pass(q.in_dtype, f.geo, ws, nelem == 0, qdiv, f.scale_out, nullptr, &f.amax_nwords, s);
            if (e != hipSuccess) return e;
        }
        const bool check = q.static_amax != nullptr;
        // per tensor, measured scale, contiguous BF16 in whole rows of
        // kTensorRowCols, no x^: the per-row kernel under the tensor's scale
        const bool tensor_rows = q.gran == G_TENSOR && q.in_dtype == D_BF16 && !q.static_amax && !q.xhat &&
                                 q.ld == q.cols && nelem > 0 && nelem % kTensorRowCols == 0;
        if (tensor_rows) {
            RowArgs r;
            r.x = q.x; r.ld = kTensorRowCols;
            r.rows = (int32_t)(nelem / kTensorRowCols); r.cpr = (int32_t)(kTensorRowCols / kChunk);
            r.codes = static_cast<uint8_t*>(q.codes); r.scales = nullptr;
            r.xhat = nullptr; r.xhat_dtype = 0; r.sink = sink;
            r.amax_words = f.amax_words; r.amax_nwords = f.amax_nwords; r.scale_out = f.scale_out;
            e = launch_row_tensor(q.fmt, r, stats, grid, s);
            stats_written = true;
        } else if (nelem || q.static_amax) {
            // static scaling launches even an empty tensor: its one workgroup
            // writes the scale derived from the caller's absmax
            e = q.in_dtype == D_BF16 ? launch_flat_fmt<D_BF16>(q.fmt, f, stats, check, grid, s)
                                     : launch_flat_fmt<D_F32>(q.fmt, f, stats, check, grid, s);
            stats_written = true;
        }
    }
    if (e != hipSuccess) return e;
    if (stats && !stats_written) {
        k_empty_stats<<<1, 64, 0, s>>>(static_cast<StatsOut*>(q.stats));
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_dequantize(const DequantArgs& d, hipStream_t s) {
    DeqArgs a;
    a.cpr = (uint32_t)(d.cols / kChunk);
    a.nchunks = (uint32_t)(d.rows * (d.cols / kChunk));
    a.cpr_shift = ilog2_exact(a.cpr);
    a.codes = static_cast<const uint8_t*>(d.codes);
    a.scales = d.scales;
    a.global_scale = d.global_scale;
    a.shifts = d.shifts;
    a.xhat = d.xhat;
    a.xhat_dtype = d.xhat_dtype;
    a.per_tensor = d.gran == G_TENSOR;
    if (a.nchunks == 0) return hipSuccess;
    const uint64_t t = tiles_of(a.nchunks);
    switch (d.fmt) {
    case F_INT8: k_dequant<F_INT8><<<grid_for(k_dequant<F_INT8>, t), kThreads, 0, s>>>(a); break;
    case F_E4M3: k_dequant<F_E4M3><<<grid_for(k_dequant<F_E4M3>, t), kThreads, 0, s>>>(a); break;
    case F_E5M2: k_dequant<F_E5M2><<<grid_for(k_dequant<F_E5M2>, t), kThreads, 0, s>>>(a); break;
    case F_MXFP4: k_dequant<F_MXFP4><<<grid_for(k_dequant<F_MXFP4>, t), kThreads, 0, s>>>(a); break;
    case F_NVFP4: k_dequant<F_NVFP4><<<grid_for(k_dequant<F_NVFP4>, t), kThreads, 0, s>>>(a); break;
    case F_INT4ZP: k_dequant<F_INT4ZP><<<grid_for(k_dequant<F_INT4ZP>, t), kThreads, 0, s>>>(a); break;
    default: k_dequant<F_INT4><<<grid_for(k_dequant<F_INT4>, t), kThreads, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

// Tiles of one launch: the grid (8 XCD slices, rounded up) stays below 2^31.
constexpr int64_t kMaxGemmTiles = ((int64_t)1 << 31) - 64;

// Token waves per workgroup: the 256-token tile from 256 tokens on.
// 256-token tiles from 1024 tokens on, and below that wherever they pad no
// more token rows than 128-token tiles do.
static int gemm_token_waves(int64_t n1) {
    const int64_t pad4 = (n1 + 255) / 256 * 256 - n1, pad2 = (n1 + 127) / 128 * 128 - n1;
    return n1 >= 1024 || (n1 >= 256 && pad4 == pad2) ? 4 : 2;
}

// z[0 .. n) = +0 (z 4-byte aligned): 16-byte stores from the first 16-byte
// boundary, single floats for the up to 3 before it and after the last.
__global__ void k_zero_f32(float* z, int64_t n) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t head = std::min<int64_t>(n, (int64_t)((16u - ((uint32_t)(uintptr_t)z & 15u)) & 15u) / 4);
    const int64_t nv = (n - head) / 4, tail0 = head + 4 * nv;
    u4v* zv = reinterpret_cast<u4v*>(z + head);
    for (int64_t i = tid; i < nv; i += stride) zv[i] = u4v{0u, 0u, 0u, 0u};
    if (tid < head) z[tid] = 0.f;
    if (tid < n - tail0) z[tail0 + tid] = 0.f;
}
static unsigned zero_grid(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n / 4 + 255) / 256, 2048)); }

hipError_t launch_zp_gemm(const ZpGemmLaunch& g, hipStream_t s) {
    if (g.n0 == 0 || g.n1 == 0) return hipSuccess;
    ZpGemmArgs a;
    a.codes = static_cast<const uint8_t*>(g.codes); a.scales = g.scales; a.shifts = g.shifts;
    a.x = static_cast<const uint16_t*>(g.x); a.z = g.z;
    a.n0 = (int32_t)g.n0; a.n1 = (int32_t)g.n1; a.K = (int32_t)g.K;
    if (g.n1 <= 32) {
        const int nt = g.n1 <= 16 ? 1 : 2, fr = g.n1 <= 8 ? 2 : 4;
        const dim3 grid((unsigned)((g.n0 + 16 * fr - 1) / (16 * fr)), (unsigned)((g.n1 + 16 * nt - 1) / (16 * nt)));
        if (g.n1 == 1) k_zp_gemv<1, true, 2><<<grid, kThreads, 0, s>>>(a);
        else if (fr == 2) k_zp_gemv<1, false, 2><<<grid, kThreads, 0, s>>>(a);
        else if (nt == 1) k_zp_gemv<1, false, 4><<<grid, kThreads, 0, s>>>(a);
        else k_zp_gemv<2, false, 4><<<grid, kThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    // up to 64 tokens: 64-token tiles (2 x 2 waves of 64 x 32, 152 registers),
    // which measured 77 us at 33-64 tokens against 104-110 us for 128-token
    // tiles; wn 1 stands for them
    const int wn = g.n1 <= 64 ? 1 : gemm_token_waves(g.n1);
    a.tiles_j = (int32_t)((g.n0 + kGemmTile - 1) / kGemmTile);
    a.tiles_n = (int32_t)((g.n1 + 64 * wn - 1) / (64 * wn));
    const int64_t tiles = (int64_t)a.tiles_j * a.tiles_n;
    // resident workgroups per CU (registers): one with 256-token tiles, two
    // with 128-token tiles, three with 64-token tiles
    const int64_t slots = 256 * (wn == 4 ? 1 : wn == 2 ? 2 : 3);
    a.ksplit = (2 * tiles <= slots && g.K >= 256) ? 2 : 1;
    const int64_t items = tiles * a.ksplit;
    if (items > kMaxGemmTiles) return hipErrorInvalidConfiguration;   // beyond one launch's grid
    a.tiles = (uint32_t)items;
    a.per_xcd = (int32_t)((items + 7) / 8);
    const unsigned grid = (unsigned)(8 * (int64_t)a.per_xcd);
    if (a.ksplit > 1) {
        const int64_t nz = g.n0 * g.n1;
        k_zero_f32<<<zero_grid(nz), 256, 0, s>>>(a.z, nz);
    }
    if (wn == 4) k_zp_gemm<256, 8><<<grid, 256 * 2, 0, s>>>(a);
    else if (wn == 2) k_zp_gemm<128, 4><<<grid, 256, 0, s>>>(a);
    else k_zp_gemm<64, 4><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_mx_gemm(const MxGemmLaunch& g, hipStream_t s) {
    if (g.n0 == 0 || g.n1 == 0) return hipSuccess;
    MxGemmArgs a;
    a.codes_w = static_cast<const uint8_t*>(g.codes_w); a.scales_w = static_cast<const uint8_t*>(g.scales_w);
    a.codes_a = static_cast<const uint8_t*>(g.codes_a); a.scales_a = static_cast<const uint8_t*>(g.scales_a);
    a.z = g.z;
    a.n0 = (int32_t)g.n0; a.n1 = (int32_t)g.n1; a.K = (int32_t)g.K;
    if (g.n1 <= 64) {
        const int nt = g.n1 <= 16 ? 1 : g.n1 <= 32 ? 2 : 4;
        const dim3 grid((unsigned)((g.n0 + 31) / 32), (unsigned)((g.n1 + 16 * nt - 1) / (16 * nt)));
        if (nt == 1) k_mx_gemv<1><<<grid, kThreads, 0, s>>>(a);
        else if (nt == 2) k_mx_gemv<2><<<grid, kThreads, 0, s>>>(a);
        else k_mx_gemv<4><<<grid, kThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    // 256 x 256 tiles with LDS DMA copies from 1024 tokens, where they fill at
    // least half of the CUs (one workgroup per CU: 136 KB of LDS); on the c3
    // weights against the 128 x 256 tiles: 1024 / 2048 / 4096 / 8192 tokens
    // 56.0 / 106.7 / 200 / 390 -> 47.4 / 94.3 / 183 / 348 us
    if (g.n1 >= 1024 && ((g.n0 + 255) / 256) * ((g.n1 + 255) / 256) >= 128) {
        a.tiles_j = (int32_t)((g.n0 + 255) / 256);
        a.tiles_n = (int32_t)((g.n1 + 255) / 256);
        const int64_t tiles = (int64_t)a.tiles_j * a.tiles_n;
        if (tiles > kMaxGemmTiles) return hipErrorInvalidConfiguration;   // beyond one launch's grid
        a.tiles = (uint32_t)tiles;
        a.per_xcd = (int32_t)((tiles + 7) / 8);
        k_mx_gemm_dma<<<(unsigned)(8 * (int64_t)a.per_xcd), 512, 0, s>>>(a);
        return hipGetLastError();
    }
    const int tn = g.n1 >= 1024 ? 256 : 128;
    // 64-row tiles where 128-row tiles would fill at most half of the CUs
    // (14336 rows up to 128 tokens: 23.2 -> 19.7 us at 65); with more tiles
    // they measured slower
    const int tm = (tn == 128 && 2 * ((g.n0 + 127) / 128) * ((g.n1 + 127) / 128) <= 256) ? 64 : 128;
    a.tiles_j = (int32_t)((g.n0 + tm - 1) / tm);
    a.tiles_n = (int32_t)((g.n1 + tn - 1) / tn);
    const int64_t tiles = (int64_t)a.tiles_j * a.tiles_n;
    if (tiles > kMaxGemmTiles) return hipErrorInvalidConfiguration;   // beyond one launch's grid
    a.tiles = (uint32_t)tiles;
    a.per_xcd = (int32_t)((tiles + 7) / 8);
    const unsigned grid = (unsigned)(8 * (int64_t)a.per_xcd);
    if (tn == 256) k_mx_gemm<256, 128><<<grid, kThreads, 0, s>>>(a);
    else if (tm == 64) k_mx_gemm<128, 64><<<grid, kThreads, 0, s>>>(a);
    else k_mx_gemm<128, 128><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_mxw_gemm(const MxwGemmLaunch& g, hipStream_t s) {
    if (g.n0 == 0 || g.n1 == 0) return hipSuccess;
    MxwGemmArgs a;
    a.codes = static_cast<const uint8_t*>(g.codes); a.scales = static_cast<const uint8_t*>(g.scales);
    a.x = static_cast<const uint16_t*>(g.x); a.z = g.z;
    a.n0 = (int32_t)g.n0; a.n1 = (int32_t)g.n1; a.K = (int32_t)g.K;
    if (g.n1 <= 64) {
        const int nt = g.n1 <= 16 ? 1 : g.n1 <= 32 ? 2 : 4, fr = (g.n1 <= 8 || nt == 4) ? 2 : 4;
        const dim3 grid((unsigned)((g.n0 + 16 * fr - 1) / (16 * fr)), (unsigned)((g.n1 + 16 * nt - 1) / (16 * nt)));
        if (g.n1 == 1) k_mxw_gemv<1, true, 2><<<grid, kThreads, 0, s>>>(a);
        else if (nt == 1 && fr == 2) k_mxw_gemv<1, false, 2><<<grid, kThreads, 0, s>>>(a);
        else if (nt == 1) k_mxw_gemv<1, false, 4><<<grid, kThreads, 0, s>>>(a);
        else if (nt == 2) k_mxw_gemv<2, false, 4><<<grid, kThreads, 0, s>>>(a);
        else k_mxw_gemv<4, false, 2><<<grid, kThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    // Grids of 128 x 128 tiles too small for two workgroups per CU take 64-row
    // tiles (1 x 4 waves of 64 x 32): twice the work items without the k
    // split's fill kernel and atomics (14336 rows, 128 tokens: 52.4 -> 41.4 us;
    // 256 tokens: 66.3 -> 60.6 us against 256-token tiles with the split)
    const int64_t rows128 = (g.n0 + 127) / 128;
    const bool small = 2 * rows128 * ((g.n1 + 127) / 128) <= 512;
    const int wn = (g.n1 >= 256 && !small) ? 4 : 2;
    const int64_t tiles128 = rows128 * ((g.n1 + 64 * wn - 1) / (64 * wn));
    const int tm = (wn == 2 && 2 * tiles128 <= 512) ? 64 : 128;
    a.tiles_j = (int32_t)((g.n0 + tm - 1) / tm);
    a.tiles_n = (int32_t)((g.n1 + 64 * wn - 1) / (64 * wn));
    // (a grid of 256-token tiles small enough to want a k split always has
    // 128 x 128 tiles few enough for this form, so no split is needed)
    // 256 x 256 tiles where the 128 x 256 tiles would take more than one
    // round of resident workgroups (c3 weights: from 768 tokens; at 384-512
    // tokens the wide tiles measured 105 against 71 us)
    const bool wide = wn == 4 && (int64_t)a.tiles_j * a.tiles_n > resident_slots(
                                     reinterpret_cast<const void*>(k_mxw_gemm<4, 128>), 512);
    if (wide) {
        a.tiles_j = (int32_t)((g.n0 + 255) / 256);
        a.tiles_n = (int32_t)((g.n1 + 255) / 256);
    }
    const int64_t tiles = (int64_t)a.tiles_j * a.tiles_n;
    if (tiles > kMaxGemmTiles) return hipErrorInvalidConfiguration;   // beyond one launch's grid
    a.tiles = (uint32_t)tiles;
    a.per_xcd = (int32_t)((tiles + 7) / 8);
    const unsigned grid = (unsigned)(8 * (int64_t)a.per_xcd);
    if (wide) k_mxw_gemm_wide<<<grid, 512, 0, s>>>(a);
    else if (wn == 4) k_mxw_gemm<4, 128><<<grid, 256 * 2, 0, s>>>(a);
    else if (tm == 64) k_mxw_gemm<2, 64><<<grid, 256, 0, s>>>(a);
    else k_mxw_gemm<2, 128><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_amax(int in_dtype, int64_t rows, int64_t cols, int64_t ld, const void* x, float* amax_out,
                       void* workspace, hipStream_t stream) {
    FlatGeom geo = make_geom(x, rows, cols, ld);
    return launch_amax_pass(in_dtype, geo, workspace, true, 0.f, nullptr, amax_out, nullptr, stream);
}

// ---------------------------------------------------------------------------
// The library's own workspace, for callers that cannot allocate: one
// file-scope device array per GPU (zero-filled when the code object loads,
// held until the process ends).  Host code never uses the array's name as
// an address: the device address comes from hipGetSymbolAddress, once per
// device with that device current, and is cached here.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static_assert(Workspace::kBytes <= kScratchBytes, "the workspace layout fits the scratch array");

hipError_t scratch_workspace(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};   // device -> address of its scratch array (no host allocation)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace iqk
