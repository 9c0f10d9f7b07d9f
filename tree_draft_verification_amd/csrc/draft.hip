// EAGLE-3 draft input fusion as two K-segmented GEMMs (news write-up of
// "EAGLE-3: Scaling up Inference Acceleration of Large Language Models via
// Training-Time Test", draft-stage paragraphs): g = W_fuse . [l; m; h] takes
// the 3k fused features to k; x = W_in . [g; E[tok]] (or [a_prev; E[tok]]
// from step 2 on, where the target's feature of an unverified token is not
// available and the draft's own output stands in) takes 2k to k. The
// embedding rows are gathered inside the GEMM's A operand.
#include "common.h"

namespace {

size_t g_bytes(int M, int k, int dtype) {
    const size_t esz = dtype == EAGLE3_BF16 ? 2 : 4;
    return ((size_t)M * k * esz + 255) & ~(size_t)255;
}

// GEMM workspace of the two FCs (K splits or tile counters; the larger)
size_t split_bytes(int M, int k, int dtype) {
    eagle3_gemm_args a{};
    a.dtype = dtype; a.M = M; a.N = k;
    a.nseg = 3; a.k[0] = a.k[1] = a.k[2] = k;
    const size_t s3 = eagle3_gemm_workspace(&a);
    a.nseg = 2; a.k[2] = 0;
    const size_t s2 = eagle3_gemm_workspace(&a);
    return s3 > s2 ? s3 : s2;
}

}  // namespace

extern "C" size_t eagle3_draft_fuse_workspace(int M, int k, int dtype) {
    if (M <= 0 || k <= 0) return 0;
    return g_bytes(M, k, dtype) + split_bytes(M, k, dtype);
}

extern "C" int eagle3_draft_fuse(const void *l, const void *m, const void *h, const void *a_prev, const int32_t *tok,
                                 const void *E, const void *w_fuse, const void *w_in, int M, int k, int V, int dtype,
                                 void *g_out, void *x_out, void *ws, size_t ws_bytes, void *stream) {
    if (M < 0 || k < 1 || V < 1) return EAGLE3_ERR_ARG;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype == EAGLE3_BF16 && k % 64 != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (M == 0) return EAGLE3_OK;
    if (!tok || !E || !w_in || !x_out) return EAGLE3_ERR_ARG;
    const bool context = a_prev == nullptr;
    if (context && (!l || !m || !h || !w_fuse)) return EAGLE3_ERR_ARG;
    if (!context && (l || m || h)) return EAGLE3_ERR_ARG;
    const void *first = a_prev;
    // the GEMMs' workspace (K splits or tile counters): after the g region
    // when g lives in the workspace, else all of it
    const size_t gb = context && !g_out ? g_bytes(M, k, dtype) : 0;
    void *split_ws = nullptr;
    size_t split_ws_bytes = 0;
    if (ws && ws_bytes > gb) {
        split_ws = (char *)ws + gb;
        split_ws_bytes = ws_bytes - gb;
    }
    if (context) {
        void *g = g_out;
        if (!g) {
            if (ws_bytes < gb || !ws) return EAGLE3_ERR_WORKSPACE;
            g = ws;
        }
        eagle3_gemm_args fa{};
        fa.dtype = dtype; fa.M = M; fa.N = k; fa.nseg = 3;
        fa.a[0] = l; fa.a[1] = m; fa.a[2] = h;
        fa.k[0] = fa.k[1] = fa.k[2] = k;
        fa.b = w_fuse; fa.c = g; fa.ldc = k;
        fa.ws = split_ws; fa.ws_bytes = split_ws_bytes;
        const int rc = eagle3_gemm(&fa, stream);
        if (rc != EAGLE3_OK) return rc;
        first = g;
    }
    eagle3_gemm_args xa{};
    xa.dtype = dtype; xa.M = M; xa.N = k; xa.nseg = 2;
    xa.a[0] = first; xa.k[0] = k;
    xa.a[1] = E; xa.a_rows[1] = tok; xa.a_nrows[1] = V; xa.k[1] = k;
    xa.b = w_in; xa.c = x_out; xa.ldc = k;
    xa.ws = split_ws; xa.ws_bytes = split_ws_bytes;
    return eagle3_gemm(&xa, stream);
}
