// Two-branch block-sparse attention forward on bf16 MFMA (gfx950).
//
// Spark-H3 page, section "Spark-Attnが変えるもの": the exact branch attends fully to the
// top-ranked key/value blocks and the compressed branch covers every other block cheaply; here the
// compressed branch is one pseudo-key per unselected block (logit s*q.k~_J + bias_J, value v~_J)
// folded into the SAME online-softmax state as the exact keys, so the branches merge exactly by
// log-sum-exp.  Core node page, section "ブロックスパースアテンション": sink_conditioning rows are
// attended exactly by every query.  H3 Optimizations README, "Nodes": non-video (sink) queries are
// dense over all keys.
//
// Design (one workgroup = one query block of BLK rows of one (batch, head); BLK/32 waves, each
// owning 32 query rows held in registers):
//  * Keys and values arrive as packed 64-key tiles (K rows | V^T, bf16, plus a log2-domain bias
//    row) written once per call by the pack kernels.  A workgroup's work is a list of tiles: its K
//    selected blocks, the sink tiles, then the compressed tiles.
//  * Tiles move HBM -> LDS with buffer_load ... lds (no register staging) into two LDS stages, the
//    K half one tile ahead of the V^T half: iteration t computes the scores of tile t+1 while it
//    turns those of tile t into probabilities and applies V(t); K(t+2) and V(t+1) stream in
//    meanwhile; one barrier per tile.  Each stage is an LDS array of its own and the loop is
//    unrolled by two, so the compiler can tell the arrays being read from those being written and
//    does not wait for the stream before LDS reads.  Two workgroups per CU hide each other's waits.
//  * A tile of real keys with no padding has an all-zero additive term: its exponents are taken
//    straight from the raw scores (one FMA per key) and its bias row is not read.
//  * LDS rows are XOR-swizzled by 16-byte chunk so the MFMA operand reads are conflict-free, and the
//    K rows of each 32-key group are loaded in the order pi (bits 2 and 3 of the row index swapped):
//    then the S^T accumulator of lane (i, h) holds, for query i, exactly the keys whose values form
//    one contiguous 16-byte chunk of a V^T row, so P feeds O^T += V^T P^T straight from registers.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: each lane holds one query's logits, so the row sum
//    needs one exchange between the wave's halves at the end.
//  * Softmax offset (FIXED pass).  A softmax is unchanged by the constant it subtracts before the
//    exponential; the running maximum of the online formulation is one choice, and a fixed value
//    known before the first tile is another (the "unified max value" of FlashDecoding++, Hong et
//    al., 2023).  Here it is a Cauchy-Schwarz bound: with q' = q * scale * log2(e) rounded to bf16
//    (the pre-scaled query the score product uses), every logit is at most
//    U = max(|q'| * kx, |q'| * kc + bc), kx the largest exact-key norm and kc, bc the largest
//    pseudo-key norm and additive term of the (batch, head).  The score accumulator starts at -U, so
//    an exact tile's probability is exp2 of the accumulator with no further arithmetic, and no
//    row maximum, exchange or rescaling runs per tile.  The bound only costs precision when the
//    row's largest logit lies far below it: a row whose normaliser comes out below 2^-64 (its
//    largest probability below 2^-64) marks its query tile, and the exact pass recomputes it.
//  * Exact pass (not FIXED).  The online formulation, run only on the marked query tiles: the
//    running max is raised when a tile's max exceeds it by more than 8 (log2 units); otherwise the
//    accumulator is not rescaled.  Probabilities are then bounded by 2^8, and the result is
//    unchanged because O and the normaliser share the max (one v_permlane32_swap per tile takes the
//    max across the wave's halves).
#include "attn_tile.hpp"

namespace spark {

constexpr float kRescaleSlack = 8.f;  // log2-domain slack before the running max is raised


// FIXED: the fixed-offset pass (writes flags[] for every query tile); otherwise the exact pass,
// which runs only the query tiles whose flag is set.
template <typename T, int D, int BLK, bool FIXED>
__global__ __launch_bounds__(BLK * 2, 2) void attn_fwd_kernel(
    const T* __restrict__ Q, const __bf16* __restrict__ packed, const float* __restrict__ bias2,
    const float4* __restrict__ bnd, int32_t* __restrict__ flags, int32_t* __restrict__ queue,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts, const int32_t* __restrict__ perm,
    T* __restrict__ O, float* __restrict__ lse, int N, int Nv, int M, int Mk, int nsh, int Ksel, int kstride, int SQ,
    int BH, int C,
    int Tv, int Ts, int Tc, float c_log2) {
// The body uses buffer resources, a device-only type: the host pass sees an empty kernel.
#if defined(__HIP_DEVICE_COMPILE__)
    using G = TileGeom<D>;
    constexpr int NT = BLK * 2;  // BLK / 32 waves
    // Each pipeline stage has LDS arrays of its own, always named statically (the stage parity is a
    // template constant), so the compiler can see that the loads streaming into one stage do not
    // write what the other stage reads, and does not wait for them before reading.
    __shared__ __attribute__((aligned(16))) __bf16 kbuf0[kTK * D];
    __shared__ __attribute__((aligned(16))) __bf16 kbuf1[kTK * D];
    __shared__ __attribute__((aligned(16))) __bf16 vbuf0[kTK * D];
    __shared__ __attribute__((aligned(16))) __bf16 vbuf1[kTK * D];
    __shared__ __attribute__((aligned(16))) float lbias0[kTK];
    __shared__ __attribute__((aligned(16))) float lbias1[kTK];
    __shared__ uint32_t sel_bits[kMaxBlocks / 32 + 2];  // + the words a padded last tile can touch
    auto kbuf = [&](auto s) __attribute__((always_inline)) -> __bf16* { if constexpr (decltype(s)::value == 0) return kbuf0; else return kbuf1; };
    auto vbuf = [&](auto s) __attribute__((always_inline)) -> __bf16* { if constexpr (decltype(s)::value == 0) return vbuf0; else return vbuf1; };
    auto lbias = [&](auto s) __attribute__((always_inline)) -> float* { if constexpr (decltype(s)::value == 0) return lbias0; else return lbias1; };

    // --- which query tile.  Sink-query tiles (dense, the longest) come first in the grid.  Video
    // query blocks are remapped so that each of the 8 XCDs (workgroup id w runs on XCD w % 8) walks
    // its own contiguous run of C query blocks of the same head while all XCDs stay on one head:
    // neighbouring query blocks select mostly the same key blocks, so concurrent workgroups of one
    // XCD share tiles in its L2, and one head's tiles are the working set of the whole chip.  In
    // the fixed-offset pass a workgroup claims the next tile of its XCD's run from a counter, and
    // once that run is spent, the next tile of another XCD's run: the XCDs do not run at one speed
    // (mean workgroup times up to 5% apart on the full clip), and the faster ones take over the
    // slower ones' last tiles instead of idling.
    // The grid holds as many video workgroups as there are (XCD, slot) items, so every workgroup
    // claims exactly one, and every item is claimed once.
    int bh, qrow0, nq, ntiles, qt;  // qt: query tile within the (batch, head): sink tiles, then video blocks
    bool dense;
    {
        const int wg = blockIdx.x;
        if (wg < BH * SQ) {
            dense = true;
            bh = wg / SQ;
            qt = wg % SQ;
            qrow0 = Nv + qt * BLK;
            nq = min(BLK, N - qrow0);
            ntiles = Tv + Ts;
        } else {
            dense = false;
            const int v = wg - BH * SQ;
            int xcd = wg & 7, slot = v >> 3;
            if constexpr (FIXED) {
                __shared__ int s_claim;
                if (threadIdx.x == 0) {
                    int c = -1;
                    for (int k = 0; k < 8 && c < 0; ++k) {
                        const int x2 = (xcd + k) & 7;
                        const int j = atomicAdd(&queue[x2], 1);
                        if (j < BH * C) c = x2 * BH * C + j;
                    }
                    s_claim = c;
                }
                __syncthreads();
                const int c = s_claim;
                if (c < 0) return;  // none left (not reached: items = workgroups); uniform
                xcd = c / (BH * C);
                slot = c % (BH * C);
            }
            bh = slot / C;
            const int I = xcd * C + slot % C;
            if (I >= M) return;  // padding slot (uniform for the workgroup, before any barrier)
            qt = SQ + I;
            qrow0 = I * BLK;
            nq = min(BLK, Nv - qrow0);
            // a variable route (counts given) lists counts[I] blocks in a row of kstride entries
            if (counts) Ksel = min(max(counts[(size_t)bh * M + I], 0), Mk);  // clamped: a bad count cannot run past the row
            ntiles = (Ksel << nsh) + Ts + Tc;
        }
    }
    int32_t* const flag = flags + (size_t)bh * (SQ + M) + qt;
    if (!FIXED && *flag == 0) return;  // left to the fixed-offset pass (uniform, before any barrier)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i32 = lane & 31, h = lane >> 5;
    const int Tall = Tv + Ts + Tc;
    const __bf16* ptile = packed + (size_t)bh * Tall * G::ELEMS;
    const float* pbias = bias2 + (size_t)bh * Tall * kTK;
    const int32_t* sel = dense ? nullptr : idx + ((size_t)bh * M + qrow0 / BLK) * kstride;
    // a selected key block is 1 << nsh tiles (key blocks of 64 or 128 keys)
    const int n_exact = dense ? 0 : Ksel << nsh;
    const int first_cmp = dense ? ntiles : n_exact + Ts;  // first compressed tile in the list

    // Selected block ids are read 64 at a time into a register (lane l holds entry base + l) and
    // taken out with readlane, so the tile loop issues no global loads besides the tile stream.  The
    // next 64 are loaded one window ahead, so moving to them never waits for memory.
    int win_base = 0, selw = 0, selw_next = 0;
    if (!dense) {
        selw = lane < Ksel ? clamp_block(sel[lane], Mk) : 0;
        selw_next = 64 + lane < Ksel ? clamp_block(sel[64 + lane], Mk) : 0;
    }
    // packed tile of list entry t (called with increasing t): selected blocks, sinks, compressed
    auto tile_of = [&](int t) __attribute__((always_inline)) -> int {
        if (dense) return t;
        if (t >= n_exact) return Tv + (t - n_exact);
        const int k = t >> nsh;
        if (k >= win_base + 64) {  // k grows by at most one per call: this is the next window
            win_base += 64;
            selw = selw_next;
            selw_next = win_base + 64 + lane < Ksel ? clamp_block(sel[win_base + 64 + lane], Mk) : 0;
        }
        return (__builtin_amdgcn_readlane(selw, k - win_base) << nsh) + (t & ((1 << nsh) - 1));
    };

    if (!dense) {
        for (int j = threadIdx.x; j < (Mk + 63) / 32 + 1; j += NT) sel_bits[j] = 0u;
        __syncthreads();
        for (int k = threadIdx.x; k < Ksel; k += NT) {
            const int J = clamp_block(sel[k], Mk);
            atomicOr(&sel_bits[J >> 5], 1u << (J & 31));
        }
    }
    using PL = DmaPlan<D, NT>;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t off_k[PL::NOFF], off_v[PL::NOFF];  // byte offsets inside a packed tile
#pragma unroll
    for (int i = 0; i < PL::NOFF; ++i) {
        off_k[i] = (uint32_t)k_src_chunk<D>(i * NT + threadIdx.x) * 16u;
        off_v[i] = (uint32_t)v_src_chunk<D>(i * NT + threadIdx.x) * 16u;
    }
    const __amdgpu_buffer_rsrc_t rs_tiles = byte_rsrc(ptile, (uint32_t)Tall * (G::ELEMS * 2));
    const __amdgpu_buffer_rsrc_t rs_bias = byte_rsrc(pbias, (uint32_t)Tall * (kTK * 4));
    // K half, V^T half plus the bias row, of packed tile tl into stage s
    auto load_k = [&](int tl, auto s) __attribute__((always_inline)) {
        issue_half<D, NT>(rs_tiles, (uint32_t)tl * (G::ELEMS * 2), off_k, kbuf(s), wv);
    };
    auto load_v = [&](int tl, auto s) __attribute__((always_inline)) {
        issue_half<D, NT>(rs_tiles, (uint32_t)tl * (G::ELEMS * 2), off_v, vbuf(s), wv);
        if (wv == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_bias, (lds_ptr)lbias(s), 4, (uint32_t)lane * 4u,
                                                     (uint32_t)tl * (kTK * 4), 0, 0);
    };
    // Pipeline: the K stream runs one tile ahead of the V stream.  Iteration t computes the scores of
    // tile t+1 (K(t+1) resident) while it turns the scores of tile t into probabilities and applies
    // V(t); K(t+2) and V(t+1) stream in meanwhile.  K(j) and V(j) live in stage j % 2.
    int tl_v;  // packed tile whose V part streams in next
    {
        const int tl0 = tile_of(0);
        load_k(tl0, IC<0>{});
        tl_v = ntiles > 1 ? tile_of(1) : 0;
        if (ntiles > 1) load_k(tl_v, IC<1>{});
        load_v(tl0, IC<0>{});
    }

    // Q rows of this wave as the B operand of S^T = K Q^T: lane (i32, h) holds row w*32 + i32,
    // dims ds*16 + 8h .. +8 for each 16-wide k step ds.  On the fixed-offset pass the row is scaled
    // into log2 units first (q * scale * log2 e, rounded to bf16), and its norm gives the offset U.
    bf16x8 qreg[D / 16];
    f32x16 sinit;  // start value of every score accumulator: 0, or -U on the fixed-offset pass
    float U = 0.f;
    {
        const int qr = w * 32 + i32;
        const T* src = Q + ((size_t)bh * N + qrow0 + qr) * D;
        float ss = 0.f;
        if constexpr (FIXED) {
            ss = load_q_scaled<T, D>(src, qr < nq, c_log2, qreg, h);
        } else {
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                u32x4 u = {0u, 0u, 0u, 0u};
                if (qr < nq) u = load8_as_bf16<T>(src + ds * 16 + 8 * h);
                qreg[ds] = __builtin_bit_cast(bf16x8, u);
            }
        }
        if constexpr (FIXED) {
            const float qn = sqrtf(ss + __shfl_xor(ss, 32));  // the row's other half is in lane i32 + 32
            const float4 bd = bnd[bh];
            U = qn * bd.x;
            if (!dense) U = fmaxf(U, fmaf(qn, bd.y, bd.z));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sinit[r] = -U;
    }

    // LDS byte offsets of this lane's MFMA operands: K rows (S^T) and V^T rows (O^T), XOR-swizzled.
    uint32_t kboff[D / 16], vboff[kTK / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) kboff[ds] = (i32 * G::CK + ((2 * ds + h) ^ swz<G::CK>(i32))) * 16;
#pragma unroll
    for (int kt = 0; kt < kTK / 16; ++kt) vboff[kt] = (i32 * G::V_CPR + ((2 * kt + h) ^ swz<G::V_CPR>(i32))) * 16;
    // A tile of real keys needs no additive term when it holds no padding: its bias row is all zero.
    const int Ns = N - Nv;
    auto clean_of = [&](int tl) __attribute__((always_inline)) -> bool {
        return tl < Tv ? (tl + 1) * kTK <= Nv : (tl - Tv + 1) * kTK <= Ns;
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // K(0), K(1), V(0) and the route bits are in LDS
    f32x16 sc[2][2];  // scores of tile t live in sc[t % 2]
    scores<D>(kbuf(IC<0>{}), kboff, qreg, sinit, sc[0]);
    bool clean_t = clean_of(tile_of(0)), clean_v = ntiles > 1 && clean_of(tl_v);  // tiles t and t+1

    // One pipeline step on stage parity P = t % 2.  MASKED: tile t is a compressed tile, whose
    // pseudo-keys of this query block's selected blocks are excluded (the mask goes into the additive
    // term with selects).
    auto step = [&](int t, auto masked, auto par, auto known_clean) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr int P = decltype(par)::value;
        __builtin_amdgcn_s_waitcnt(0);  // this thread's share of K(t+1), V(t) has landed
        __syncthreads();                // ... everyone's; K(t) and V(t-1) buffers are free
        const int tl_k = t + 2 < ntiles ? tile_of(t + 2) : 0;
        if (t + 2 < ntiles) load_k(tl_k, IC<P>{});
        if (t + 1 < ntiles) load_v(tl_v, IC<P ^ 1>{});
        const bool clean = decltype(known_clean)::value || (!MASKED && clean_t);
        clean_t = clean_v;
        clean_v = t + 2 < ntiles && clean_of(tl_k);
        tl_v = tl_k;
        scores<D>(kbuf(IC<P ^ 1>{}), kboff, qreg, sinit, sc[P ^ 1]);  // tile t+1 (unused after the last)

        // ---- probabilities of tile t.  Register 4g+j of chunk c holds key c*32 + 16(g/2) + 8h + 4(g%2) + j.
        f32x16 (&st)[2] = sc[P];
        float cc = 1.f, neg_m = 0.f;  // exponent of key j: x_j * cc + neg_m
        if constexpr (FIXED) {
            // x = q'.k - U (the accumulator), plus the additive term on tiles that carry one
            if (!clean) {
                const int cbase = (t - first_cmp) * kTK;  // first pseudo-key of a compressed tile
                const float* lb = lbias(IC<P>{});
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int key = c * 32 + 16 * (g >> 1) + 8 * h + 4 * (g & 1);
                        f32x4 bb = *reinterpret_cast<const f32x4*>(lb + key);
                        if constexpr (MASKED) {
                            const uint32_t selw_ = sel_bits[(cbase + key) >> 5] >> ((cbase + key) & 31);
#pragma unroll
                            for (int j = 0; j < 4; ++j) bb[j] = ((selw_ >> j) & 1u) ? -INFINITY : bb[j];
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) st[c][4 * g + j] += bb[j];
                    }
            }
        } else {
            // Exponent: x_j * cc - m with x the raw score (cc = scale*log2 e) on a tile without an
            // additive term, else x = raw*scale*log2 e + bias (cc = 1).
            float mx = -INFINITY;
            if (clean) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[c][r]);
                mx = half_max(mx) * c_log2;  // scale > 0: the max commutes with it
                cc = c_log2;
            } else {
                const int cbase = (t - first_cmp) * kTK;  // first pseudo-key of a compressed tile
                const float* lb = lbias(IC<P>{});
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int key = c * 32 + 16 * (g >> 1) + 8 * h + 4 * (g & 1);
                        f32x4 bb = *reinterpret_cast<const f32x4*>(lb + key);
                        if constexpr (MASKED) {
                            const uint32_t selw_ = sel_bits[(cbase + key) >> 5] >> ((cbase + key) & 31);
#pragma unroll
                            for (int j = 0; j < 4; ++j) bb[j] = ((selw_ >> j) & 1u) ? -INFINITY : bb[j];
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            st[c][4 * g + j] = fmaf(st[c][4 * g + j], c_log2, bb[j]);
                            mx = fmaxf(mx, st[c][4 * g + j]);
                        }
                    }
                mx = half_max(mx);
            }
            const bool raise = mx > m_run + kRescaleSlack;
            if (__ballot(raise)) {
                const float m_new = raise ? mx : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
                m_run = m_new;
            }
            neg_m = m_run == -INFINITY ? 0.f : -m_run;
        }
        // P in bf16, 16 keys per PV step: lane (i32, h) supplies keys 16kt + 8h + e (e = 0..7).
        // The normaliser sums the same bf16 values the PV product uses.
        const char* Vb = reinterpret_cast<const char*>(vbuf(IC<P>{}));
        // The probability/PV phase runs at raised wave priority: the SIMD's other wave is then most
        // often in its score or row-max phase, so the two keep both the VALU and the matrix pipe fed.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kt = 0; kt < kTK / 16; ++kt) {
            bf16x8 pk;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pk[e] = (__bf16)__builtin_amdgcn_exp2f(FIXED ? st[kt >> 1][8 * (kt & 1) + e]
                                                             : fmaf(st[kt >> 1][8 * (kt & 1) + e], cc, neg_m));
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 pr = {pk[e], pk[e + 1]};
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
            }
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {  // V^T row dt*32 + i32 is 64*kTK bytes past row i32
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vb + dt * 64 * kTK + vboff[kt]);
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk, acc[dt], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // Steps over [t, end) with the stage parity a template constant: pairs (even, odd), plus one
    // step at either end when the range starts odd or ends early.
    auto run = [&](int t, int end, auto masked) __attribute__((always_inline)) {
        constexpr std::false_type any{};
        if (t < end && (t & 1)) step(t++, masked, IC<1>{}, any);
        if constexpr (!decltype(masked)::value) {
            // leading pairs of tiles known to need no additive term (all but ragged edge tiles)
            for (; t + 1 < end && clean_t && clean_v; t += 2) {
                step(t, masked, IC<0>{}, std::true_type{});
                step(t + 1, masked, IC<1>{}, std::true_type{});
            }
        }
        for (; t + 1 < end; t += 2) {
            step(t, masked, IC<0>{}, any);
            step(t + 1, masked, IC<1>{}, any);
        }
        if (t < end) step(t++, masked, IC<0>{}, any);
        return t;
    };
    run(run(0, first_cmp, std::false_type{}), ntiles, std::true_type{});

    // ---- epilogue: lane (i32, h) holds query row w*32 + i32, dims dt*32 + 8*g + 4*h + (0..3)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    const int qr = w * 32 + i32;
    if constexpr (FIXED) {
        // the offset U lay too far above this row's logits: the exact pass redoes the query tile
        // (written for every tile on every call, so the flags need no clearing)
        const int under = __syncthreads_or(qr < nq && !(l_tot >= 0x1p-64f));
        if (threadIdx.x == 0) *flag = under;
        if (under) return;
        m_run = U;
    }
    if (qr < nq) {
        const int row = qrow0 + qr;
        const int orow = (!dense && perm) ? perm[(size_t)bh * Nv + row] : row;
        if (!dense && perm && (unsigned)orow >= (unsigned)Nv) return;  // a permutation entry out of range: row not written
        T* dst = O + ((size_t)bh * N + orow) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = dt * 32 + 8 * g + 4 * h;
                if constexpr (sizeof(T) == 2) {
                    bf16x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = (__bf16)(acc[dt][4 * g + j] * inv);
                    *reinterpret_cast<bf16x4*>(dst + col) = o;
                } else {
                    f32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = acc[dt][4 * g + j] * inv;
                    *reinterpret_cast<f32x4*>(dst + col) = o;
                }
            }
        if (lse && h == 0) lse[(size_t)bh * N + orow] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
    }
#endif
}

// The fixed-offset pass's tile counters start at zero on every call (a kernel, not a memset, so
// that a captured graph replays it).
__global__ __launch_bounds__(64) void attn_queue_zero_kernel(int32_t* __restrict__ queue) {
    if (threadIdx.x < 8) queue[threadIdx.x] = 0;
}

template <typename T, int D, int BLK>
static void launch_attend_t(const LaunchCtx& L, const void* Q, const void* packed, const int32_t* idx,
                            const int32_t* counts, const int32_t* perm, void* O, float* lse) {
    const PackGeom g = pack_geom(L);
    const int SQ = g.SQ;
    const int C = (L.M + 7) / 8;  // query blocks per XCD per head
    const dim3 grid(L.BH * SQ + L.BH * 8 * C);
    const float c_log2 = L.scale * 1.4426950408889634f;
    const char* pk = (const char*)packed;
    const float* b2 = (const float*)(pk + g.bias_off);
    const float4* bnd = (const float4*)(pk + g.bnd_off);
    int32_t* flags = (int32_t*)(pk + g.flag_off);  // workspace the library owns inside the packed buffer
    int32_t* queue = (int32_t*)(pk + g.queue_off);  // likewise
    const int nsh = L.block_k == 128 ? 1 : 0, kstride = counts ? L.Mk : L.K;
    // fixed-offset pass over every query tile, then the exact pass over the tiles it marked
    hipLaunchKernelGGL(attn_queue_zero_kernel, dim3(1), dim3(64), 0, L.stream, queue);
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BLK, true>), grid, dim3(BLK * 2), 0, L.stream, (const T*)Q,
                       (const __bf16*)packed, b2, bnd, flags, queue, idx, counts, perm, (T*)O, lse, L.N, L.Nv, L.M, L.Mk,
                       nsh, L.K, kstride, SQ, L.BH, C, g.Tv, g.Ts, g.Tc, c_log2);
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BLK, false>), grid, dim3(BLK * 2), 0, L.stream, (const T*)Q,
                       (const __bf16*)packed, b2, bnd, flags, nullptr, idx, counts, perm, (T*)O, lse, L.N, L.Nv, L.M, L.Mk,
                       nsh, L.K, kstride, SQ, L.BH, C, g.Tv, g.Ts, g.Tc, c_log2);
}

void launch_attend(const LaunchCtx& L, const void* Q, const void* packed, const int32_t* idx, const int32_t* counts,
                   const int32_t* perm, void* O, float* lse) {
#define SPARK_ATTN_CASE(T, D, B)                                          \
    if (L.d == D && L.block == B) {                                       \
        launch_attend_t<T, D, B>(L, Q, packed, idx, counts, perm, O, lse); \
        return;                                                           \
    }
    if (L.dtype == SPARK_ATTN_BF16) {
        SPARK_ATTN_CASE(__bf16, 64, 64) SPARK_ATTN_CASE(__bf16, 64, 128)
        SPARK_ATTN_CASE(__bf16, 128, 64) SPARK_ATTN_CASE(__bf16, 128, 128)
    } else {
        SPARK_ATTN_CASE(float, 64, 64) SPARK_ATTN_CASE(float, 64, 128)
        SPARK_ATTN_CASE(float, 128, 64) SPARK_ATTN_CASE(float, 128, 128)
    }
#undef SPARK_ATTN_CASE
}

}  // namespace spark
