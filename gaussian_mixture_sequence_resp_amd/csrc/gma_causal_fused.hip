// Causal GMA forward with the responsibilities kept on chip (bf16 inputs, gfx950).
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283), "Core mechanism" item 3: position i
// reads the inclusive prefix of the latent memory and normaliser,
//     O_i = gamma_Q,i . S_i / (gamma_Q,i . z_i + eps),   [S_i | z_i] = sum_{j <= i} gamma_K,j (x) [v_j | 1],
// with gamma the GMM posterior of item 1 (the five-pass split logit contraction of
// gma_mfma_common.h, then the softmax over the K components).
//
// Component-parallel layout.  A workgroup has eight waves; wave w owns the 32 components
// 32 w .. 32 w + 31 (K padded to 256) and keeps their bf16 hi/lo coefficient fragments and c_k
// in registers for the whole kernel (128 < K <= 256), so no coefficient block is staged in LDS and the
// responsibilities never go to HBM.  The sequence of a head is walked in groups of 32
// positions; per group:
//   logits   every wave: its 32 x 32 logit tiles of the group's queries and keys (operands:
//            the group's routing rows split exactly into x, x2 hi, x2 lo, staged in LDS once);
//   softmax  every wave publishes, per position and side, the maximum of its 32 logits and the
//            sum of 2^(l - that maximum); after one barrier each wave combines the eight pairs
//            (M = max, s = sum of ps_w 2^(pm_w - M)) and scales its exponentials by
//            2^(pm_w - M) / s: the normalised responsibilities, bf16, into LDS;
//   outputs  waves 0..NT: Gamma_Q [S | z] against the bf16 shadow of the state entering the
//            group (one output tile each: value tiles, then the normaliser tile); wave NT+1: the
//            intra-group affinity Gamma_K Gamma_Q^T, zero above the diagonal (positions after i
//            cannot reach O_i); after a barrier the value waves add affinity x [V | 1];
//   update   every wave: its state tiles (its components x [value dims | 1], fp32 in
//            registers) += Gamma_K^T [V | 1] over the group, then its part of the bf16 shadow;
//            waves 4..7, which hold no output tile, also stage the next group's rows (the
//            exact x^2 split into LDS) and load the rows of the group after it.
// The sequence of a head is cut into segments that run in parallel; the state entering a
// segment is the ordered sum of the totals Gamma_K^T [V | 1] of the sub-segments before it,
// which the same kernel computes in its totals mode (key side only) beforehand.
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_common.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {
namespace mf {
namespace {

constexpr int kFWaves = 8;                 // waves per workgroup = component tiles of 32
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFKp = 32 * kFWaves;         // components (padded) covered by one workgroup
constexpr int kGrp = 32;                   // positions per group
constexpr int kModeScan = 0, kModeTotals = 1;

// LDS layout of one workgroup (byte offsets).
template <int NC, int NTS>
struct FLds {
    static constexpr int Dvs = 32 * NTS;
    static constexpr int XS = 2 * NC * 3 * 1024;  // routing operands: [side][chunk][x, x2h, x2l][64 lanes][16 B]
    static constexpr int GS = 2 * kFKp + 16;      // responsibilities row stride: [side][position][component]
    static constexpr int GB = 2 * kGrp * GS;
    static constexpr int SS = 2 * kFKp + 16;      // state shadow row stride
    static constexpr int SB = (Dvs + 32) * SS;    // S^T (Dvs rows), z hi (8), z lo (8), ones (16)
    static constexpr int VS = 2 * Dvs + 32;       // value rows of a group: [position][dim]
    static constexpr int VB = kGrp * VS;
    static constexpr int XCH = 2 * kGrp * kFWaves * 8;  // [side][position][wave] (max, sum)
    static constexpr int AFF = 2 * 64 * 16;              // packed affinity operand, 2 fragments
    static constexpr int DEN = kGrp * 4;
    static constexpr int CK = kFKp * 4;                  // c_k of the head
    static constexpr int DUMMY = 16;                     // target of the stores of threads without a vector
    static constexpr int xs0 = 0, xs1 = XS, g = 2 * XS, sh = g + GB, v0 = sh + SB, v1 = v0 + VB, xch = v1 + VB,
                         aff = xch + XCH, den = aff + AFF, ck = den + DEN, dummy = ck + CK, total = dummy + DUMMY;
};

// This thread's share of a group's routing rows: one 16-byte vector (side, chunk, lane) for
// threads < 128 NC, loaded into registers two groups ahead and stored into LDS as the exact
// split x, x2 hi, x2 lo (the logits' B operands) one group ahead.
template <int NC>
struct XRows {
    bf16x8 x;
    // branch-free (so that the loads and stores can be scheduled among MFMAs): threads past the
    // NC x 128 vectors read a valid row and store into a dummy LDS slot; dims past d_r are zeroed
    __device__ __forceinline__ void load(const bf16_t* q_h, const bf16_t* k_h, int p0, int N, int dr, bool keys_only) {
        const int t = threadIdx.x % (128 * NC);
        const int side = t / (64 * NC), rem = t % (64 * NC), c = rem / 64, lane = rem % 64;
        const int pos = min(p0 + (lane & 31), N - 1), d0 = 16 * c + 8 * (lane >> 5);
        const bool in = d0 < dr;
        const bf16_t* src = (side == 0 && !keys_only ? q_h : k_h) + (size_t)pos * dr + (in ? d0 : 0);
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(src);
        const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        x = in ? val : z;
    }
    __device__ __forceinline__ void store(unsigned char* xs, unsigned char* dummy) const {
        const int t = threadIdx.x;
        const int side = (t / (64 * NC)) & 1, rem = t % (64 * NC), c = rem / 64, lane = rem % 64;
        XFrag f;
        f.x1 = x;
        split_square(f);
        unsigned char* dst = t < 128 * NC ? xs + ((size_t)(side * NC + c) * 3) * 1024 + 16 * lane : dummy;
        const int step = t < 128 * NC ? 1024 : 0;
        *reinterpret_cast<bf16x8*>(dst) = f.x1;
        *reinterpret_cast<bf16x8*>(dst + step) = f.x2h;
        *reinterpret_cast<bf16x8*>(dst + 2 * step) = f.x2l;
    }
};

// This thread's share of a group's value rows (position, 8 dims) for threads < 4 Dvs, loaded one
// group ahead of being stored into LDS (row-major [position][dim], stride 2 Dvs + 32 bytes).
template <int NTS>
struct VRows {
    static constexpr int Dvs = 32 * NTS;
    bf16x8 v;
    // branch-free as XRows: threads past the 4 Dvs vectors read a valid row and store into the
    // dummy slot; dims past d_v are zeroed
    __device__ __forceinline__ void load(const bf16_t* v_h, int p0, int N, int dv) {
        const int t = threadIdx.x % (4 * Dvs);
        const int pos = min(p0 + t / (Dvs / 8), N - 1), d0 = 8 * (t % (Dvs / 8));
        const bool in = d0 < dv;
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(v_h + (size_t)pos * dv + (in ? d0 : 0));
        const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        v = in ? val : z;
    }
    __device__ __forceinline__ void store(unsigned char* sV, unsigned char* dummy) const {
        constexpr int VSt = 2 * Dvs + 32;
        const int t = threadIdx.x;
        unsigned char* dst = t < 4 * Dvs ? sV + (size_t)(t / (Dvs / 8)) * VSt + 16 * (t % (Dvs / 8)) : dummy;
        *reinterpret_cast<bf16x8*>(dst) = v;
    }
};

// The same staging done by the waves 4..7 alone (256 threads, index ts): XV vectors of
// routing rows and one of value rows per thread.  In the scan these waves have the least work
// after the responsibilities are in LDS (the output tiles are on waves 0..NTS+1), so the next
// group's rows are split, stored and the following group's loaded there.
template <int NC>
struct XRowsW {
    static constexpr int XV = (128 * NC + 255) / 256;
    bf16x8 x[XV];
    __device__ __forceinline__ void load(const bf16_t* q_h, const bf16_t* k_h, int p0, int N, int dr, int ts) {
#pragma unroll
        for (int e = 0; e < XV; ++e) {
            const int t = (ts + 256 * e) % (128 * NC);
            const int side = t / (64 * NC), rem = t % (64 * NC), c = rem / 64, lane = rem % 64;
            const int pos = min(p0 + (lane & 31), N - 1), d0 = 16 * c + 8 * (lane >> 5);
            const bool in = d0 < dr;
            const bf16_t* src = (side == 0 ? q_h : k_h) + (size_t)pos * dr + (in ? d0 : 0);
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(src);
            const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
            x[e] = in ? val : z;
        }
    }
    __device__ __forceinline__ void store(unsigned char* xs, unsigned char* dummy, int ts) const {
#pragma unroll
        for (int e = 0; e < XV; ++e) {
            const int tt = ts + 256 * e;
            const int t = tt % (128 * NC);
            const int side = t / (64 * NC), rem = t % (64 * NC), c = rem / 64, lane = rem % 64;
            XFrag f;
            f.x1 = x[e];
            split_square(f);
            const bool real = tt < 128 * NC;
            unsigned char* dst = real ? xs + ((size_t)(side * NC + c) * 3) * 1024 + 16 * lane : dummy;
            const int step = real ? 1024 : 0;
            *reinterpret_cast<bf16x8*>(dst) = f.x1;
            *reinterpret_cast<bf16x8*>(dst + step) = f.x2h;
            *reinterpret_cast<bf16x8*>(dst + 2 * step) = f.x2l;
        }
    }
};

template <int NTS>
struct VRowsW {
    static constexpr int Dvs = 32 * NTS;
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16_t* v_h, int p0, int N, int dv, int ts) {
        const int t = ts % (4 * Dvs);
        const int pos = min(p0 + t / (Dvs / 8), N - 1), d0 = 8 * (t % (Dvs / 8));
        const bool in = d0 < dv;
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(v_h + (size_t)pos * dv + (in ? d0 : 0));
        const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        v = in ? val : z;
    }
    __device__ __forceinline__ void store(unsigned char* sV, unsigned char* dummy, int ts) const {
        constexpr int VSt = 2 * Dvs + 32;
        unsigned char* dst = ts < 4 * Dvs ? sV + (size_t)(ts / (Dvs / 8)) * VSt + 16 * (ts % (Dvs / 8)) : dummy;
        *reinterpret_cast<bf16x8*>(dst) = v;
    }
};

// Logits of one side of the group for this wave's 32 components, C[k][t]: seed_logits sets
// c_k (register 4q + r: component 32 w + 8 q + 4 half + r), chunk_logits adds one 16-wide
// chunk c of routing dims (the five passes ah.x2h, bh.x, al.x2h, bl.x, ah.x2l).
__device__ __forceinline__ void seed_logits(f32x16& acc, const float* sCk) {
    const float* cv = sCk + 32 * wave_id() + 4 * (lane_id() >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 c4 = *reinterpret_cast<const float4*>(cv + 8 * q);
        acc[4 * q] = c4.x;
        acc[4 * q + 1] = c4.y;
        acc[4 * q + 2] = c4.z;
        acc[4 * q + 3] = c4.w;
    }
}

__device__ __forceinline__ void chunk_logits(f32x16& acc, const bf16x8 (&cf)[4], const unsigned char* xs_chunk) {
    const unsigned char* src = xs_chunk + 16 * lane_id();
    const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(src);
    const bf16x8 x2h = *reinterpret_cast<const bf16x8*>(src + 1024);
    const bf16x8 x2l = *reinterpret_cast<const bf16x8*>(src + 2048);
    // pieces: 0 ah, 1 al, 2 bh, 3 bl
    acc = mfma(cf[0], x2h, acc);
    acc = mfma(cf[2], x1, acc);
    acc = mfma(cf[1], x2h, acc);
    acc = mfma(cf[3], x1, acc);
    acc = mfma(cf[0], x2l, acc);
}

template <int NC>
__device__ __forceinline__ f32x16 group_logits(const bf16x8 (&cf)[NC][4], const float* sCk,
                                               const unsigned char* xs_side) {
    f32x16 acc;
    seed_logits(acc, sCk);
#pragma unroll
    for (int c = 0; c < NC; ++c) chunk_logits(acc, cf[c], xs_side + (size_t)c * 3 * 1024);
    return acc;
}

// Bf16 shadow of this wave's state tiles (components 32 w .., value tile n) for the next
// group's Gamma_Q [S | z]: S^T rows, and z as hi (rows Dvs..Dvs+7) and lo (Dvs+8..Dvs+15).
template <int NTS>
__device__ __forceinline__ void shadow_tiles(unsigned char* sS, int ss, const f32x16 (&st)[NTS + 1],
                                             unsigned char* dummy) {
    constexpr int Dvs = 32 * NTS;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
#pragma unroll
    for (int n = 0; n <= NTS; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k0 = 32 * w + 8 * q + 4 * half;
            const float v0 = st[n][4 * q], v1 = st[n][4 * q + 1], v2 = st[n][4 * q + 2], v3 = st[n][4 * q + 3];
            if (n < NTS) {
                *reinterpret_cast<uint2*>(sS + (size_t)(32 * n + col) * ss + 2 * k0) =
                    make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
            } else {
                // lanes 0..7 write z hi rows, 8..15 z lo rows; the others (whose rows hold the
                // constant ones) write the dummy slot: a store for every lane, no branch
                uint2 hi, lo;
                hi.x = pack_bf16(v0, v1);
                hi.y = pack_bf16(v2, v3);
                lo.x = pack_bf16(v0 - bf16lo_to_f32(hi.x), v1 - bf16hi_to_f32(hi.x));
                lo.y = pack_bf16(v2 - bf16lo_to_f32(hi.y), v3 - bf16hi_to_f32(hi.y));
                unsigned char* dst = col < 16 ? sS + (size_t)(Dvs + col) * ss + 2 * k0 : dummy;
                *reinterpret_cast<uint2*>(dst) = col < 8 ? hi : lo;
            }
        }
}

// MODE kModeScan: one workgroup per (head, segment): outputs of the segment's positions.
// MODE kModeTotals: one workgroup per (head, sub-segment): Gamma_K^T [V | 1] of its positions
// into tpart (fp32 rows k of Dvs + 1 columns).  W, cvec: coefficients of gma_prep (Kp = 256).
template <int NC, int NTS, int MODE>
__global__ void __launch_bounds__(kFThreads, 2)
    gma_causal_fused(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ kr, const bf16_t* __restrict__ v,
                     const bf16_t* __restrict__ W, const float* __restrict__ cvec, float* __restrict__ tpart,
                     bf16_t* __restrict__ out, float eps, int BH, int H, int N, int dr, int dv, int seg_len,
                     int nseg, int nsub_per_seg, int nsub) {
    extern __shared__ __align__(16) unsigned char smem[];
    using L = FLds<NC, NTS>;
    constexpr int Dvs = L::Dvs, Dp = 16 * NC;
    constexpr int KS = kFKp / 16;  // 16-wide contraction steps over the components
    constexpr bool kScan = MODE == kModeScan;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;

    int bh, part;
    head_part(blockIdx.x, BH, kScan ? nseg : nsub, bh, part);
    const int h = bh % H;
    const int sub_len = kScan ? seg_len : seg_len / nsub_per_seg;
    const int n_begin = part * sub_len;
    const int n_end = min(N, n_begin + sub_len);
    const bf16_t* q_h = qr + (size_t)bh * N * dr;
    const bf16_t* k_h = kr + (size_t)bh * N * dr;
    const bf16_t* v_h = v + (size_t)bh * N * dv;

    // ---- this wave's coefficient fragments (registers, whole kernel); c_k of the head in LDS
    bf16x8 cf[NC][4];
    {
        const bf16_t* wrow = W + ((size_t)h * kFKp + 32 * w + col) * 4 * Dp + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int p = 0; p < 4; ++p) cf[c][p] = *reinterpret_cast<const bf16x8*>(wrow + p * Dp + 16 * c);
        if ((int)threadIdx.x < kFKp)
            reinterpret_cast<float*>(smem + L::ck)[threadIdx.x] = cvec[(size_t)h * kFKp + threadIdx.x];
    }
    const float* sCk = reinterpret_cast<const float*>(smem + L::ck);

    // ---- state tiles (components 32 w .., value tile n; n = NTS is z in every column): the
    // carry entering a scan segment is the ordered sum of the sub-segment totals before it
    f32x16 st[NTS + 1];
#pragma unroll
    for (int n = 0; n <= NTS; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) st[n][e] = 0.0f;
    if (kScan) {
        const size_t per = (size_t)kFKp * (Dvs + 1);
        const float* src = tpart + (size_t)bh * nsub * per;
        const int nprev = part * nsub_per_seg;
        for (int u = 0; u < nprev; ++u) {
            const float* p = src + (size_t)u * per;
#pragma unroll
            for (int n = 0; n <= NTS; ++n) {
                const int cc = n < NTS ? 32 * n + col : Dvs;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    st[n][e] += p[(size_t)(32 * w + 8 * (e >> 2) + 4 * half + (e & 3)) * (Dvs + 1) + cc];
            }
        }
    }
    unsigned char* sG = smem + L::g;
    unsigned char* sS = smem + L::sh;
    float* xch = reinterpret_cast<float*>(smem + L::xch);
    if (kScan) {
        // constant rows of the shadow: ones (rows Dvs+16 .. Dvs+31), then the carry
        for (int i = threadIdx.x; i < 16 * (kFKp / 8); i += kFThreads) {
            bf16x8 o8;
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = (short)0x3f80;
            *reinterpret_cast<bf16x8*>(sS + (size_t)(Dvs + 16 + i / (kFKp / 8)) * L::SS + 16 * (i % (kFKp / 8))) = o8;
        }
        shadow_tiles<NTS>(sS, L::SS, st, smem + L::dummy);
    }

    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (short)0x3f80;
    constexpr int S0 = kScan ? 0 : 1;  // first side: queries (scan) or keys only (totals)

    // local softmax statistics of one side's logits tile (lg <- 2^(lg - pm), this wave's 32
    // components), published as (pm, ps) for every position
    auto local_stats = [&](f32x16& t, int side) {
        float pm = t[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) pm = fmaxf(pm, t[i]);
        pm = max_halves(pm);
        // a tile of padded components only (the last one when K <= 224) has every logit -inf:
        // its exponentials are 0 against any finite shift
        const float sh = pm == -INFINITY ? 0.0f : pm;
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(t[i] - sh);
            t[i] = e;
            ps += e;
        }
        ps = sum_halves(ps);
        // both lane halves hold the same pair: both store it (no branch)
        *reinterpret_cast<float2*>(xch + ((size_t)(side * kGrp + col) * kFWaves + w) * 2) = make_float2(pm, ps);
    };
    // the eight waves' statistics combined (M = max, s = sum of ps_u 2^(pm_u - M)); this wave's
    // exponentials scaled by 2^(pm_w - M) / s: its normalised responsibilities, bf16, into LDS
    auto assemble = [&](const f32x16& t, int side, bool valid) {
        // lanes l and l + 32 hold the same position: each half takes four waves' pairs, then
        // the halves exchange (maximum, then the two partial sums)
        constexpr int WH = kFWaves / 2;
        const float4* xp = reinterpret_cast<const float4*>(xch + (size_t)(side * kGrp + col) * kFWaves * 2) +
                           (WH / 2) * half;
        float pmv[WH], psv[WH];
#pragma unroll
        for (int u = 0; u < WH / 2; ++u) {
            const float4 a4 = xp[u];
            pmv[2 * u] = a4.x;
            psv[2 * u] = a4.y;
            pmv[2 * u + 1] = a4.z;
            psv[2 * u + 1] = a4.w;
        }
        float M = pmv[0];
#pragma unroll
        for (int u = 1; u < WH; ++u) M = fmaxf(M, pmv[u]);
        M = max_halves(M);
        float ssum = 0.0f;
#pragma unroll
        for (int u = 0; u < WH; ++u) ssum += psv[u] * fast_exp2(pmv[u] - M);
        ssum = sum_halves(ssum);
        // this wave's own maximum (a uniform LDS offset, not a dynamic register index)
        const float pmw = xch[((size_t)(side * kGrp + col) * kFWaves + w) * 2];
        // positions past the segment (keys) must not enter the state: zero responsibility
        // (a multiply, not a branch: this code is scheduled among MFMAs)
        const float f = fast_exp2(pmw - M) / ssum * (valid ? 1.0f : 0.0f);
        unsigned char* grow = sG + (size_t)(side * kGrp + col) * L::GS;
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
            const int i0 = 8 * qp;
            auto sx = __builtin_amdgcn_permlane32_swap(pack_bf16(t[i0] * f, t[i0 + 1] * f),
                                                       pack_bf16(t[i0 + 4] * f, t[i0 + 5] * f), false, false);
            auto sy = __builtin_amdgcn_permlane32_swap(pack_bf16(t[i0 + 2] * f, t[i0 + 3] * f),
                                                       pack_bf16(t[i0 + 6] * f, t[i0 + 7] * f), false, false);
            *reinterpret_cast<uint4*>(grow + 2 * (32 * w + 16 * qp + 8 * half)) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
        }
    };

    const int ngroups = n_end > n_begin ? (n_end - n_begin + kGrp - 1) / kGrp : 0;
    XRows<NC> xr;
    VRows<NTS> vr;
    XRowsW<NC> xw;
    VRowsW<NTS> vw;
    const bool stager = w >= kFWaves / 2;
    const int ts = (int)threadIdx.x - kFThreads / 2;
    // group 0's rows staged, group 1's in flight (scan: by the waves 4..7)
    if (ngroups > 0) {
        if constexpr (kScan) {
            if (stager) {
                xw.load(q_h, k_h, n_begin, N, dr, ts);
                vw.load(v_h, n_begin, N, dv, ts);
                xw.store(smem + L::xs0, smem + L::dummy, ts);
                vw.store(smem + L::v0, smem + L::dummy, ts);
                xw.load(q_h, k_h, n_begin + kGrp, N, dr, ts);
                vw.load(v_h, n_begin + kGrp, N, dv, ts);
            }
        } else {
            xr.load(q_h, k_h, n_begin, N, dr, !kScan);
            vr.load(v_h, n_begin, N, dv);
            xr.store(smem + L::xs0, smem + L::dummy);
            vr.store(smem + L::v0, smem + L::dummy);
            xr.load(q_h, k_h, n_begin + kGrp, N, dr, !kScan);
            vr.load(v_h, n_begin + kGrp, N, dv);
        }
    }
    __syncthreads();
    bf16x8 den_ones;  // normaliser tile of the intra term: ones in rows 0..7 (the z hi rows)
#pragma unroll
    for (int j = 0; j < 8; ++j) den_ones[j] = (short)(col < 8 ? 0x3f80 : 0);

    for (int g = 0; g < ngroups; ++g) {
        const int p0 = n_begin + g * kGrp;
        const unsigned char* xs = smem + ((g & 1) ? L::xs1 : L::xs0);
        const unsigned char* sV = smem + ((g & 1) ? L::v1 : L::v0);
        // ---- logits of both sides (keys only in totals mode), local softmax statistics
        f32x16 lg[2];
#pragma unroll
        for (int side = S0; side < 2; ++side) {
            lg[side] = group_logits<NC>(cf, sCk, xs + (size_t)side * NC * 3 * 1024);
            local_stats(lg[side], side);
        }
        lds_barrier();  // ---- 1: statistics of all waves published
        // ---- normalised responsibilities into LDS; the next group's rows staged, the one after
        // that loaded
#pragma unroll
        for (int side = S0; side < 2; ++side) assemble(lg[side], side, side == 0 || p0 + col < n_end);
        if constexpr (!kScan) {
            xr.store(smem + ((g & 1) ? L::xs0 : L::xs1), smem + L::dummy);
            vr.store(smem + ((g & 1) ? L::v0 : L::v1), smem + L::dummy);
            xr.load(q_h, k_h, p0 + 2 * kGrp, N, dr, !kScan);
            vr.load(v_h, p0 + 2 * kGrp, N, dv);
        }
        lds_barrier();  // ---- 2: responsibilities of the group in LDS
        const unsigned char* gq = sG;
        const unsigned char* gk = sG + (size_t)kGrp * L::GS;
        f32x16 o;
        if (kScan) {
            if (w <= NTS) {
                // Gamma_Q [S | z] for output tile n = w (A: shadow rows, B: Gamma_Q)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[i] = 0.0f;
                const unsigned char* arow = sS + (size_t)(32 * w + col) * L::SS + 16 * half;
                const unsigned char* brow = gq + (size_t)col * L::GS + 16 * half;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    o = mfma(*reinterpret_cast<const bf16x8*>(arow + 32 * ks),
                             *reinterpret_cast<const bf16x8*>(brow + 32 * ks), o);
            } else if (w == NTS + 1) {
                // intra-group affinity A[j][i] = gamma_K,j . gamma_Q,i, zero for j > i
                f32x16 aff;
#pragma unroll
                for (int i = 0; i < 16; ++i) aff[i] = 0.0f;
                const unsigned char* arow = gk + (size_t)col * L::GS + 16 * half;
                const unsigned char* brow = gq + (size_t)col * L::GS + 16 * half;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    aff = mfma(*reinterpret_cast<const bf16x8*>(arow + 32 * ks),
                               *reinterpret_cast<const bf16x8*>(brow + 32 * ks), aff);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int jrow = 8 * (i >> 2) + 4 * half + (i & 3);
                    aff[i] = (jrow <= col) ? aff[i] : 0.0f;
                }
                bf16x8* ap = reinterpret_cast<bf16x8*>(smem + L::aff);
                ap[l] = pack8(aff, 0, 1.0f);
                ap[64 + l] = pack8(aff, 8, 1.0f);
            }
        }
        // state += Gamma_K^T [V | 1] over the group (this wave's components)
#pragma unroll
        for (int ks = 0; ks < kGrp / 16; ++ks) {
            const bf16x8 a = lds_frag_tr(gk, L::GS, 16 * ks, 32 * w);
#pragma unroll
            for (int n = 0; n <= NTS; ++n) {
                const bf16x8 b = n < NTS ? lds_frag_tr(sV, L::VS, 16 * ks, 32 * n) : ones;
                st[n] = mfma(a, b, st[n]);
            }
        }
        if (!kScan) {
            lds_barrier();  // ---- everyone done with this group's responsibilities
            continue;
        }
        if (stager) {
            // the next group's rows (into the buffers group g - 1 used), the one after loaded
            xw.store(smem + ((g & 1) ? L::xs0 : L::xs1), smem + L::dummy, ts);
            vw.store(smem + ((g & 1) ? L::v0 : L::v1), smem + L::dummy, ts);
            xw.load(q_h, k_h, p0 + 2 * kGrp, N, dr, ts);
            vw.load(v_h, p0 + 2 * kGrp, N, dv, ts);
        }
        lds_barrier();  // ---- 3: affinity in LDS; the old shadow is no longer read
        if (w <= NTS) {
            const bf16x8* ap = reinterpret_cast<const bf16x8*>(smem + L::aff);
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
                const bf16x8 b = ap[64 * sh + l];
                const bf16x8 a = w < NTS ? lds_frag_tr_crows(sV, L::VS, 16 * sh, 32 * w) : den_ones;
                o = mfma(a, b, o);
            }
            // both lane halves hold the same normaliser: both store it (no branch)
            if (w == NTS) reinterpret_cast<float*>(smem + L::den)[col] = o[0] + o[4];
        }
        shadow_tiles<NTS>(sS, L::SS, st, smem + L::dummy);
        lds_barrier();  // ---- 4: normaliser and new shadow in LDS
        if (w < NTS) {
            const int t = p0 + col;
            const float inv = 1.0f / (reinterpret_cast<const float*>(smem + L::den)[col] + eps);
            bf16_t* orow = out + ((size_t)bh * N + t) * dv;
#pragma unroll
            for (int qp = 0; qp < 2; ++qp) {
                uint2 q0, q1;
                q0.x = pack_bf16(o[8 * qp] * inv, o[8 * qp + 1] * inv);
                q0.y = pack_bf16(o[8 * qp + 2] * inv, o[8 * qp + 3] * inv);
                q1.x = pack_bf16(o[8 * qp + 4] * inv, o[8 * qp + 5] * inv);
                q1.y = pack_bf16(o[8 * qp + 6] * inv, o[8 * qp + 7] * inv);
                auto sx = __builtin_amdgcn_permlane32_swap(q0.x, q1.x, false, false);
                auto sy = __builtin_amdgcn_permlane32_swap(q0.y, q1.y, false, false);
                const int d0 = 32 * w + 16 * qp + 8 * half;
                if (t < n_end && d0 < dv) *reinterpret_cast<uint4*>(orow + d0) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
            }
        }
    }

    if (!kScan) {
        float* T = tpart + ((size_t)bh * nsub + part) * kFKp * (Dvs + 1);
#pragma unroll
        for (int n = 0; n <= NTS; ++n)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k = 32 * w + 8 * (e >> 2) + 4 * half + (e & 3);
                if (n < NTS)
                    T[(size_t)k * (Dvs + 1) + 32 * n + col] = st[n][e];
                else if (col == 0)
                    T[(size_t)k * (Dvs + 1) + Dvs] = st[n][e];
            }
    }
}

struct FusedLayout {
    size_t W, C, tpart, total;
    int S, seg_len, TS, nsub;
};

FusedLayout fused_layout(const gma_desc& d) {
    const Geo g = geometry(d);
    const int BH = d.B * d.H;
    FusedLayout L;
    const int groups = (d.N + kGrp - 1) / kGrp;
    int s = (256 + BH - 1) / BH;
    if (s > groups) s = groups;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    L.seg_len = ((d.N + s - 1) / s + kGrp - 1) / kGrp * kGrp;
    L.S = (d.N + L.seg_len - 1) / L.seg_len;
    if (L.S < 1) L.S = 1;
    // totals: every segment before the last cut into TS equal sub-segments so that about
    // 256 workgroups run; TS divides the segment's group count
    const int seg_groups = L.seg_len / kGrp;
    L.TS = 1;
    if (L.S > 1) {
        const int want = (256 + BH * (L.S - 1) - 1) / (BH * (L.S - 1));
        for (int t = 1; t <= seg_groups && t <= want; ++t)
            if (seg_groups % t == 0) L.TS = t;
    }
    L.nsub = (L.S - 1) * L.TS;
    size_t off = 0;
    L.W = off;
    off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
    L.C = off;
    off += align_up((size_t)d.H * g.Kp * sizeof(float));
    L.tpart = off;
    off += align_up((size_t)BH * (L.nsub > 0 ? L.nsub : 1) * g.Kp * (g.Dvp + 1) * sizeof(float));
    L.total = off;
    return L;
}

typedef void (*FusedFn)(const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*, const float*, float*, bf16_t*,
                        float, int, int, int, int, int, int, int, int, int);

template <int NC, int NTS>
bool fused_pick(FusedFn& scan, FusedFn& tot) {
    scan = gma_causal_fused<NC, NTS, kModeScan>;
    tot = gma_causal_fused<NC, NTS, kModeTotals>;
    return true;
}

bool fused_select(const Geo& g, FusedFn& scan, FusedFn& tot) {
    if (g.NT == 1) {
        switch (g.NC) {
            case 1: return fused_pick<1, 1>(scan, tot);
            case 2: return fused_pick<2, 1>(scan, tot);
            case 4: return fused_pick<4, 1>(scan, tot);
        }
    } else if (g.NT == 2) {
        switch (g.NC) {
            case 1: return fused_pick<1, 2>(scan, tot);
            case 2: return fused_pick<2, 2>(scan, tot);
            case 4: return fused_pick<4, 2>(scan, tot);
        }
    }
    return false;
}

size_t fused_lds(const Geo& g) {
    switch (g.NT * 8 + g.NC) {
        case 8 + 1: return FLds<1, 1>::total;
        case 8 + 2: return FLds<2, 1>::total;
        case 8 + 4: return FLds<4, 1>::total;
        case 16 + 1: return FLds<1, 2>::total;
        case 16 + 2: return FLds<2, 2>::total;
        case 16 + 4: return FLds<4, 2>::total;
    }
    return 0;
}

}  // namespace

// 128 < K <= 256 (eight component tiles), d_r <= 64, d_v <= 64, bf16 with dims multiples of 8.
bool fused_causal_supported(const gma_desc& d) {
    if (d.dtype != GMA_BF16 || d.d_r % 8 != 0 || d.d_v % 8 != 0) return false;
    const Geo g = geometry(d);
    FusedFn s, t;
    return g.MT == kFWaves && fused_select(g, s, t) && fused_lds(g) <= kLdsMax;
}

size_t fused_causal_workspace(const gma_desc& d) { return fused_layout(d).total; }

hipError_t fused_causal_forward(const Args& a) {
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const FusedLayout L = fused_layout(d);
    bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
    float* cvec = reinterpret_cast<float*>(a.ws + L.C);
    float* tpart = reinterpret_cast<float*>(a.ws + L.tpart);
    const int BH = d.B * d.H;
    FusedFn scan, tot;
    if (!fused_select(g, scan, tot)) return hipErrorNotSupported;
    hipError_t e;
    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;
    const size_t lds = fused_lds(g);
    const bf16_t* q = static_cast<const bf16_t*>(a.qr);
    const bf16_t* k = static_cast<const bf16_t*>(a.kr);
    const bf16_t* v = static_cast<const bf16_t*>(a.v);
    bf16_t* o = static_cast<bf16_t*>(a.out);
    if (L.nsub > 0) {
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(tot), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds)) != hipSuccess)
            return e;
        rec_begin(a, "gma_causal_fused_totals");
        hipLaunchKernelGGL(tot, dim3(BH * L.nsub), dim3(kFThreads), lds, a.stream, q, k, v, W, cvec, tpart, o, a.eps,
                           BH, d.H, d.N, d.d_r, d.d_v, L.seg_len, L.S, L.TS, L.nsub);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
        return e;
    rec_begin(a, "gma_causal_fused_scan");
    hipLaunchKernelGGL(scan, dim3(BH * L.S), dim3(kFThreads), lds, a.stream, q, k, v, W, cvec, tpart, o, a.eps, BH,
                       d.H, d.N, d.d_r, d.d_v, L.seg_len, L.S, L.TS, L.nsub);
    rec_end(a);
    return hipGetLastError();
}

}  // namespace mf
}  // namespace gma
