// Shared definitions of the gfx950 kernels: compiled shape, vector types,
// bf16/fp16 helpers, and the fixed permutation of K inside 8-element blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Compiled layer shape ("Config" table of the qwen35moe forward-pass page).
constexpr int D = 2048;   // n_embd
constexpr int E = 256;    // routed experts
constexpr int K = 8;      // experts used per token
constexpr int F = 512;    // routed expert FF
constexpr int FS = 512;   // shared expert FF
constexpr int G = 64;     // quantisation group
constexpr int WAVE = 64;

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// A finite fp32 value as two bf16: hi = v truncated to bf16 (never
// overflows), lo = the remainder v - hi (exact in fp32) rounded to bf16.
// hi + lo carries 16 significant bits of v (|v - hi - lo| <= 2^-16 |v|) with
// the whole fp32 range, so intermediates stored this way cannot overflow
// where fp16 would.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    const uint32_t h = __float_as_uint(v) & 0xffff0000u;
    hi = (uint16_t)(h >> 16);
    lo = f32_to_bf16_rne(v - __uint_as_float(h));
}

// Nearest bf16 of a finite double, ties to even: round to fp32 by truncation
// with a sticky last bit (round to odd: 24 bits keep what the second rounding
// needs), then to bf16 to nearest even.  One correct rounding overall.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
    const float f = (float)d;
    uint32_t u = __float_as_uint(f);
    const double back = (double)f;
    if (back != d) {
        if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1;  // one fp32 ulp toward zero
        u |= 1u;
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Double sum over the 64 lanes of a wave by a fixed xor butterfly: every lane
// ends with the same, order-fixed value.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// K order inside every 8-element block of an fp16 operand row.  Position p
// holds element kPerm8[p] = {0,4,1,5,2,6,3,7}[p]: the order in which one u32
// of eight nibbles unpacks into four fp16 pairs (nibbles j and j+4 land in
// one 32-bit lane).  Every fp16 GEMM operand (activations and dequantised
// weights) uses this order, so dot products over K are unchanged.
__host__ __device__ constexpr int perm8_pos(int j) { return j < 4 ? 2 * j : 2 * (j - 4) + 1; }

// Eight bf16 (natural order, 4 dwords) -> eight fp16 in perm8 order.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_perm(u32x4 v) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        f16x2 p = {(f16)f[j], (f16)f[j + 4]};
        o[j] = __builtin_bit_cast(uint32_t, p);
    }
    return o;
}

// One u32 of eight nibbles -> four dwords of 16-bit patterns (magic byte,
// nibble) in perm8 order: dword j holds nibbles j and j + 4 in its low and
// high halves.  `magic4` holds the magic byte in all four bytes (0x64: fp16
// 1024 + q; 0x43: bf16 128 + q).  The even and odd nibbles are masked into
// bytes once; v_perm_b32 then places two of them beside two magic bytes per
// dword (7 VALU ops per word instead of 11 for shift, mask and or per pair).
__device__ __forceinline__ u32x4 nibble_codes(uint32_t w, uint32_t magic4) {
    const uint32_t ev = w & 0x0f0f0f0fu;         // bytes: nibbles 0, 2, 4, 6
    const uint32_t od = (w >> 4) & 0x0f0f0f0fu;  // bytes: nibbles 1, 3, 5, 7
    // selector bytes 0..3 pick the second operand's bytes, 4..7 the first's
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(magic4, ev, 0x04020400u);  // nibbles 0, 4
    o[1] = __builtin_amdgcn_perm(magic4, od, 0x04020400u);  // nibbles 1, 5
    o[2] = __builtin_amdgcn_perm(magic4, ev, 0x04030401u);  // nibbles 2, 6
    o[3] = __builtin_amdgcn_perm(magic4, od, 0x04030401u);  // nibbles 3, 7
    return o;
}

// One u32 of eight 4-bit codes -> eight fp16 weights s*q + b (one rounding,
// fused multiply-add) in perm8 order.  s2, b2 hold the group's scale and
// bias in both halves.
__device__ __forceinline__ u32x4 q4_word_to_f16x8(uint32_t w, f16x2 s2, f16x2 b2) {
    const f16x2 k1024 = {(f16)1024.0f, (f16)1024.0f};
    const u32x4 c = nibble_codes(w, 0x64646464u);  // fp16 1024 + q: the 10-bit mantissa holds q exactly
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t cj = c[j];
        f16x2 q = __builtin_bit_cast(f16x2, cj) - k1024;  // exact
        f16x2 r = __builtin_elementwise_fma(q, s2, b2);
        o[j] = __builtin_bit_cast(uint32_t, r);
    }
    return o;
}

// ---- Power-of-two row exponents of the fp16 MFMA operands.
//
// Every fp16 operand row (activations, dequantised or converted weights,
// intermediates) is stored as v * 2^-e with e chosen from the row's largest
// magnitude m so that m * 2^-e lies in [2^14, 2^15): no finite input
// overflows the fp16 range, values down to 2^-28 m keep their full 11-bit
// significand, and the exponents are re-applied exactly (ldexp) in fp32.
// An all-zero row gets EXP_ZERO, below any real exponent, so it never
// dominates a maximum of exponents.
constexpr int EXP_ZERO = -1000;
__device__ __forceinline__ int row_exp(float m) {
    if (!(m > 0.0f)) return EXP_ZERO;
    int e;
    __builtin_frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
    return e - 15;
}

// Largest value of a non-negative float over each 16-lane row (every lane
// of the row gets it); and over each half-wave of 32 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_fmax_step(float v) {
    return __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float row16_max(float v) {
    v = dpp_fmax_step<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_fmax_step<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_fmax_step<0x141>(v);  // row_half_mirror
    v = dpp_fmax_step<0x140>(v);  // row_mirror
    return v;
}
__device__ __forceinline__ float half32_max(float v) {
    v = row16_max(v);
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);  // rows 0<->1, 2<->3
    return __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}

// Eight fp32 values (natural order) scaled by 2^-e -> eight fp16 in the
// perm8 order (pairs j, j + 4), each rounded once.
__device__ __forceinline__ u32x4 f32x8_to_f16x8_perm_scaled(const float* v, int e) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const f16x2 p = {(f16)__builtin_ldexpf(v[j], -e), (f16)__builtin_ldexpf(v[j + 4], -e)};
        o[j] = __builtin_bit_cast(uint32_t, p);
    }
    return o;
}

// fp16 2^d for d <= 0 (0 below the smallest subnormal, 2^-24): the factor
// that moves a row piece stored with exponent e_piece to the row's largest
// exponent e_max, d = e_piece - e_max.  Multiplying fp16 values by it is
// exact while the result stays normal; what falls below is under 2^-25 of
// the row's largest value.
__device__ __forceinline__ f16 pow2_f16(int d) {
    return d < -24 ? (f16)0.0f : (f16)__builtin_ldexpf(1.0f, d);
}

// Raw buffer resource over an array of at most 2 GiB (no stride, bounds
// check at 2^31 - 1 bytes); offsets are bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, 0x00020000);
}
// The same array with no bytes in range: a load through it returns zeros
// and reaches no memory (the range check drops it), so a load ring can be
// fed past its last unit without fetching anything.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t empty_rsrc(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0, 0x00020000);
}

// silu(z) = z * sigmoid(z) with the hardware exp2 and reciprocal (about
// 1 ulp each): every caller rounds the result to fp16 or feeds an fp32 dot
// product, far coarser than the few-ulp difference from an IEEE division.
// z -> -inf: exp overflows to inf and the reciprocal to 0, giving -0.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Signed-integer key with the order of a float that is not NaN: the bits
// as they are for v >= 0, the magnitude bits flipped for v < 0; -0 becomes
// +0 first, so equal keys mean equal floats.
__device__ __forceinline__ int order_key(float v) {
    const int b = __builtin_bit_cast(int, v + 0.0f);
    return b ^ ((b >> 31) & 0x7fffffff);
}

// Wave-wide maximum of an int, the same value in every lane: row maxima
// through DPP, then rows (0,1) and (2,3) through v_permlane16_swap and the
// halves through v_permlane32_swap.
template <int CTRL>
__device__ __forceinline__ int dpp_max_step(int v) {
    return max(v, __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ int wave_max(int v) {
    v = dpp_max_step<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_step<0x141>(v);  // row_half_mirror
    v = dpp_max_step<0x140>(v);  // row_mirror
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    v = max((int)p[0], (int)p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return max((int)q[0], (int)q[1]);
}

// Wave-wide minimum of an int, the same value in every lane (as wave_max).
template <int CTRL>
__device__ __forceinline__ int dpp_min_step(int v) {
    return min(v, __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ int wave_min(int v) {
    v = dpp_min_step<0xB1>(v);
    v = dpp_min_step<0x4E>(v);
    v = dpp_min_step<0x141>(v);
    v = dpp_min_step<0x140>(v);
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    v = min((int)p[0], (int)p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return min((int)q[0], (int)q[1]);
}

// The float an order key stands for (order_key inverted; -0 comes back +0).
// v + the value lane CTRL names (0 where there is none or the row is masked)
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add_from(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, true);
}
// inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 within each
// row of 16, then lane 15 into rows 1 and 3, lane 31 into rows 2 and 3
__device__ __forceinline__ int wave_incl_scan(int v) {
    v = dpp_add_from<0x111, 0xf>(v);
    v = dpp_add_from<0x112, 0xf>(v);
    v = dpp_add_from<0x114, 0xf>(v);
    v = dpp_add_from<0x118, 0xf>(v);
    v = dpp_add_from<0x142, 0xa>(v);
    v = dpp_add_from<0x143, 0xc>(v);
    return v;
}

__device__ __forceinline__ float key_float(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7fffffff)); }

// Top-8 of 256 scores held by one wave (lane l holds experts l, l+64,
// l+128, l+192 in v[0..3]), ordered by (score desc, index asc); the scores
// are finite or -inf, never NaN.  Each lane sorts its four candidates once,
// as order keys; in each of the eight rounds the winner is then the lowest
// index among the lane heads equal to the wave maximum (a lane's other
// candidates equal to it would sit behind a head of the same score and a
// lower index).  A round takes the wave maximum of the heads' keys and a
// ballot of the heads that equal it: one such head wins outright, equal
// maxima in several lanes go to the lowest index (a wave minimum).  The
// winning lane, known by its lane number, shifts its list by selects, so a
// round's chain is the maximum, one ballot and the selects.
// The results are wave-uniform.  Only the first `rounds` ranks are formed
// (wave-uniform, 1..8); later entries of sel_v / sel_i are left unset.
__device__ __forceinline__ void wave_top8(const float* v, int lane, float* sel_v, int* sel_i, int rounds = 8) {
    int k[4], ai[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
        k[c] = order_key(v[c]);
        ai[c] = lane + 64 * c;
    }
    // sort the lane's four candidates (compare-exchange network; equal keys
    // keep index order)
    const int net[5][2] = {{0, 1}, {2, 3}, {0, 2}, {1, 3}, {1, 2}};
#pragma unroll
    for (int s = 0; s < 5; s++) {
        const int p = net[s][0], q = net[s][1];
        const bool sw = (k[q] > k[p]) | ((k[q] == k[p]) & (ai[q] < ai[p]));
        const int tk = k[p], ti = ai[p];
        k[p] = sw ? k[q] : k[p];
        ai[p] = sw ? ai[q] : ai[p];
        k[q] = sw ? tk : k[q];
        ai[q] = sw ? ti : ai[q];
    }
    // a lane that has given all four holds INT_MIN, below the key of -inf
#pragma unroll
    for (int r = 0; r < 8; r++) {
        if (r >= rounds) break;
        const int mk = wave_max(k[0]);
        const uint64_t at_max = __ballot(k[0] == mk);
        int wl;
        if (__popcll(at_max) == 1) {
            wl = __ffsll((unsigned long long)at_max) - 1;
        } else {  // equal maxima in several lanes: the lowest index wins
            const int mi = wave_min(k[0] == mk ? ai[0] : 0x7fffffff);
            wl = __ffsll((unsigned long long)__ballot(ai[0] == mi)) - 1;
        }
        sel_v[r] = key_float(mk);
        sel_i[r] = __builtin_amdgcn_readlane(ai[0], wl);
        const bool win = lane == wl;  // this lane gave the winner: shift its list
        k[0] = win ? k[1] : k[0];
        ai[0] = win ? ai[1] : ai[0];
        k[1] = win ? k[2] : k[1];
        ai[1] = win ? ai[2] : ai[1];
        k[2] = win ? k[3] : k[2];
        ai[2] = win ? ai[3] : ai[2];
        k[3] = win ? (int)0x80000000 : k[3];
        ai[3] = win ? 0x7fffffff : ai[3];
    }
}

// The experts of one token and their logits (lrow: the token's E logits),
// wave-uniform in sel_i / sel_v: the top K by logit (wave_top8), or with a
// hash table (ds4.c study notes Part 3, MoE trace 3: experts looked up by
// token id in a precomputed [K, n_vocab] table) column `tok` of the table in
// table order.  The id and the entries are clamped into range.  A caller
// that needs only the first `ranks` experts may say so: the top-K selection
// then stops there (the table form sets all K regardless).
// HASH is a compile-time choice so that the top-K path carries no trace of
// the table path.
template <bool HASH>
__device__ __forceinline__ void select_experts(const float* lrow, const int32_t* tid2eid, int n_vocab, int tok,
                                               int lane, float* sel_v, int* sel_i, int ranks = K) {
    if constexpr (HASH) {
        tok = min(max(tok, 0), n_vocab - 1);
        const int e = min(max(tid2eid[(size_t)min(lane, K - 1) * n_vocab + tok], 0), E - 1);
        const float v = lrow[e];
#pragma unroll
        for (int r = 0; r < K; r++) {
            sel_i[r] = __builtin_amdgcn_readlane(e, r);
            sel_v[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), r));
        }
    } else {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; c++) v[c] = lrow[lane + 64 * c];
        wave_top8(v, lane, sel_v, sel_i, ranks);
    }
}

// Sum over each 16-lane row; every lane of the row ends with the same,
// order-fixed value (each step adds a lane's partner, and the partner adds
// the same two terms).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v = quad_sum(v);
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    return v;
}

// Largest of the K selected logits: the first one of a top-K selection,
// any of them for a table's.
template <bool HASH>
__device__ __forceinline__ float selected_max(const float* sel_v) {
    float m = sel_v[0];
    if constexpr (HASH) {
#pragma unroll
        for (int r = 1; r < K; r++) m = __builtin_fmaxf(m, sel_v[r]);
    }
    return m;
}

// Routing score of a selected logit v given the largest selected one v0, before the
// renormalisation over the top k: softmax exp(v - v0) (the full-softmax
// normaliser cancels), or sqrt(softplus(v)), softplus computed stably
// (log1p(e^v); v beyond +-20 is v or e^v to fp32 precision, and sqrt(e^v)
// is e^(v/2)).  When even the top logit is below -20, every selected score
// is e^(v/2) and the common factor e^(v0/2) cancels in the renormalisation:
// the scores are taken as e^((v - v0)/2), which no logit underflows.
__device__ __forceinline__ float route_score(float v, float v0, int gating) {
    if (gating == 0) return __expf(v - v0);
    if (v < -20.0f) return __expf(0.5f * (v0 < -20.0f ? v - v0 : v));
    return __builtin_sqrtf(v > 20.0f ? v : log1pf(__expf(v)));
}

// Sum over the 64 lanes of a wave, the same value in every lane: row sums,
// then rows (0,1) and (2,3) through v_permlane16_swap, then the two halves
// through v_permlane32_swap.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    v = __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
    const uint32_t c = __builtin_bit_cast(uint32_t, v);
    const auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
    return __builtin_bit_cast(float, (uint32_t)q[0]) + __builtin_bit_cast(float, (uint32_t)q[1]);
}

}  // namespace moe
