// Argument validation (pure host C++).
#include "validate.hpp"

namespace fp8bq {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool fmt_ok(int f) { return f == 0 || f == 1; }
static int in_esize(int t) { return t == 0 ? 2 : (t == 1 ? 4 : 0); }

// No device allocation reaches 2^48 bytes; bounding every matrix's byte extent by that keeps the
// extent and overlap arithmetic below free of overflow.
constexpr int64_t kMaxExtentBytes = int64_t(1) << 48;

int check_mat(const Mat& m, bool align_ld) {
  if (m.p == nullptr) return kErrNull;
  if (!aligned16(m.p)) return kErrAlign;
  if (m.ld < m.cols || m.ld < 1) return kErrLd;
  const int64_t max_elems = kMaxExtentBytes / m.esize;
  if (m.ld > max_elems || (m.rows > 1 && m.rows - 1 > (max_elems - m.cols) / m.ld)) return kErrShape;
  if (align_ld && ((m.ld * m.esize) % 16) != 0) return kErrLd;
  return kOk;
}

static void extent(const Mat& m, uintptr_t& lo, uintptr_t& hi) {
  lo = (uintptr_t)m.p;
  hi = lo + (uintptr_t)(((m.rows - 1) * m.ld + m.cols) * m.esize);
}

bool overlaps(const Mat& a, const Mat& b) {
  if (a.rows <= 0 || a.cols <= 0 || b.rows <= 0 || b.cols <= 0) return false;
  uintptr_t alo, ahi, blo, bhi;
  extent(a, alo, ahi);
  extent(b, blo, bhi);
  return alo < bhi && blo < ahi;
}

// Common tail of the three quantizers: input X, codes Q, scales S (each a Mat), checked in order.
static int check_quant(const Mat& x, const Mat& q, const Mat& s, bool s_align) {
  int st;
  if (x.p == nullptr || q.p == nullptr || s.p == nullptr) return kErrNull;
  if ((st = check_mat(x, true)) != kOk) return st;
  if ((st = check_mat(q, true)) != kOk) return st;
  if ((st = check_mat(s, s_align)) != kOk) return st;
  if (overlaps(q, x) || overlaps(s, x) || overlaps(q, s)) return kErrOverlap;
  return kOk;
}

int validate_quant_1x128(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, const void* q,
                         int64_t ldq, const void* s, int64_t lds, bool* empty) {
  *empty = false;
  if (in_esize(xt) == 0) return kErrDtype;
  if (!fmt_ok(fmt)) return kErrFormat;
  if (R < 0 || C < 0 || C % 128 != 0) return kErrShape;
  if (R == 0 || C == 0) {
    *empty = true;
    return kOk;
  }
  return check_quant(Mat{x, R, C, ldx, in_esize(xt)}, Mat{q, R, C, ldq, 1}, Mat{s, C / 128, R, lds, 4}, true);
}

int validate_quant_128x1(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, const void* qt,
                         int64_t ldqt, const void* st, int64_t ldst, bool* empty) {
  *empty = false;
  if (in_esize(xt) == 0) return kErrDtype;
  if (!fmt_ok(fmt)) return kErrFormat;
  if (R < 0 || C < 0 || R % 128 != 0 || C % 8 != 0) return kErrShape;
  if (R == 0 || C == 0) {
    *empty = true;
    return kOk;
  }
  return check_quant(Mat{x, R, C, ldx, in_esize(xt)}, Mat{qt, C, R, ldqt, 1}, Mat{st, R / 128, C, ldst, 4}, true);
}

int validate_quant_dual(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fr, const void* q, int64_t ldq,
                        const void* s, int64_t lds, int fc, const void* qt, int64_t ldqt, const void* st,
                        int64_t ldst, bool* empty) {
  *empty = false;
  if (in_esize(xt) == 0) return kErrDtype;
  if (!fmt_ok(fr) || !fmt_ok(fc)) return kErrFormat;
  if (R < 0 || C < 0 || R % 128 != 0 || C % 128 != 0) return kErrShape;
  if (R == 0 || C == 0) {
    *empty = true;
    return kOk;
  }
  const Mat mx{x, R, C, ldx, in_esize(xt)};
  const Mat mq{q, R, C, ldq, 1}, ms{s, C / 128, R, lds, 4};
  const Mat mqt{qt, C, R, ldqt, 1}, mst{st, R / 128, C, ldst, 4};
  int r;
  if ((r = check_quant(mx, mq, ms, true)) != kOk) return r;
  if ((r = check_quant(mx, mqt, mst, true)) != kOk) return r;
  if (overlaps(mq, mqt) || overlaps(mq, mst) || overlaps(ms, mqt) || overlaps(ms, mst)) return kErrOverlap;
  return kOk;
}

int validate_quant_128x128_dual(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, const void* q,
                                int64_t ldq, const void* s, int64_t lds, const void* qt, int64_t ldqt, bool* empty) {
  *empty = false;
  if (in_esize(wt) == 0) return kErrDtype;
  if (!fmt_ok(fmt)) return kErrFormat;
  if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return kErrShape;
  if (N == 0 || K == 0) {
    *empty = true;
    return kOk;
  }
  const Mat mw{w, N, K, ldw, in_esize(wt)}, mq{q, N, K, ldq, 1}, ms{s, N / 128, K / 128, lds, 4};
  const Mat mqt{qt, K, N, ldqt, 1};
  int r;
  if ((r = check_quant(mw, mq, ms, false)) != kOk) return r;
  if (qt == nullptr) return kErrNull;
  if ((r = check_mat(mqt, true)) != kOk) return r;
  if (overlaps(mqt, mw) || overlaps(mqt, mq) || overlaps(mqt, ms)) return kErrOverlap;
  return kOk;
}

int validate_quant_128x128(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, const void* q,
                           int64_t ldq, const void* s, int64_t lds, bool* empty) {
  *empty = false;
  if (in_esize(wt) == 0) return kErrDtype;
  if (!fmt_ok(fmt)) return kErrFormat;
  if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return kErrShape;
  if (N == 0 || K == 0) {
    *empty = true;
    return kOk;
  }
  return check_quant(Mat{w, N, K, ldw, in_esize(wt)}, Mat{q, N, K, ldq, 1}, Mat{s, N / 128, K / 128, lds, 4},
                     false);
}

int validate_quant_weights_dual(const WeightJobArgs* jobs, int count, int max_jobs, int wt, int fmt, bool* empty) {
  if (count < 0 || count > max_jobs) return kErrValue;
  if (count > 0 && jobs == nullptr) return kErrNull;
  int r;
  for (int j = 0; j < count; ++j) {
    const WeightJobArgs& a = jobs[j];
    if ((r = validate_quant_128x128_dual(a.w, wt, a.N, a.K, a.ldw, fmt, a.q, a.ldq, a.s, a.lds, a.qt, a.ldqt,
                                         &empty[j])) != kOk)
      return r;
  }
  const int es = in_esize(wt);
  for (int i = 0; i < count; ++i) {
    if (empty[i]) continue;
    const WeightJobArgs& a = jobs[i];
    const Mat outs[3] = {{a.q, a.N, a.K, a.ldq, 1}, {a.s, a.N / 128, a.K / 128, a.lds, 4}, {a.qt, a.K, a.N, a.ldqt, 1}};
    for (int j = 0; j < count; ++j) {
      if (j == i || empty[j]) continue;
      const WeightJobArgs& b = jobs[j];
      const Mat theirs[4] = {{b.w, b.N, b.K, b.ldw, es},
                             {b.q, b.N, b.K, b.ldq, 1},
                             {b.s, b.N / 128, b.K / 128, b.lds, 4},
                             {b.qt, b.K, b.N, b.ldqt, 1}};
      for (const Mat& o : outs)
        for (const Mat& t : theirs)
          if (overlaps(o, t)) return kErrOverlap;
    }
  }
  return kOk;
}

static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int validate_quant_tensor(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, const void* amax,
                          double beta, const void* q, int64_t ldq, const void* qt, int64_t ldqt, const void* s,
                          const void* ws, size_t ws_bytes, size_t ws_needed, bool* empty) {
  *empty = false;
  if (in_esize(xt) == 0) return kErrDtype;
  if (!fmt_ok(fmt)) return kErrFormat;
  if (!(beta >= 0.0 && beta <= 1.0)) return kErrValue;  // also rejects NaN
  if (R < 0 || C < 0 || C % 128 != 0 || (qt != nullptr && R % 128 != 0)) return kErrShape;
  if (R == 0 || C == 0) {
    *empty = true;
    return kOk;
  }
  // ws_needed == 0: the caller passes no workspace (the kernels use the library's own scratch)
  const bool has_ws = ws_needed > 0;
  if (x == nullptr || q == nullptr || amax == nullptr || s == nullptr || (has_ws && ws == nullptr)) return kErrNull;
  int st;
  const Mat mx{x, R, C, ldx, in_esize(xt)}, mq{q, R, C, ldq, 1}, mqt{qt, C, R, ldqt, 1};
  const Mat ma{amax, 1, 1, 1, 4}, ms{s, 1, 1, 1, 4};
  if ((st = check_mat(mx, true)) != kOk) return st;
  if ((st = check_mat(mq, true)) != kOk) return st;
  if (qt != nullptr && (st = check_mat(mqt, true)) != kOk) return st;
  if (!aligned4(amax) || !aligned4(s) || (has_ws && !aligned16(ws))) return kErrAlign;
  if (ws_bytes < ws_needed) return kErrWorkspace;
  const Mat mw{has_ws ? ws : nullptr, 1, (int64_t)ws_needed, (int64_t)ws_needed, 1};
  const Mat outs[4] = {mq, mqt, ma, ms};
  const int nout = 4;
  for (int i = 0; i < nout; ++i) {
    if (outs[i].p == nullptr) continue;
    if (overlaps(outs[i], mx) || (has_ws && overlaps(outs[i], mw))) return kErrOverlap;
    for (int j = i + 1; j < nout; ++j)
      if (outs[j].p != nullptr && overlaps(outs[i], outs[j])) return kErrOverlap;
  }
  if (has_ws && overlaps(mw, mx)) return kErrOverlap;
  return kOk;
}

static bool finite_nonneg(double v) { return v >= 0.0 && v <= 1.7976931348623157e308; }

int validate_hyperball(const void* w, int64_t ldw, const void* g, int gt, int64_t ldg, int64_t R, int64_t C,
                       double lr, double wd, double eps, double radius, const void* norms, const void* ws,
                       size_t ws_bytes, size_t ws_needed, bool* empty) {
  *empty = false;
  if (in_esize(gt) == 0) return kErrDtype;
  if (!finite_nonneg(lr) || !finite_nonneg(wd) || !finite_nonneg(radius) || !(finite_nonneg(eps) && eps > 0.0))
    return kErrValue;
  if (R < 0 || C < 0 || C % 8 != 0) return kErrShape;
  if (R == 0 || C == 0) {
    *empty = true;
    return kOk;
  }
  if (w == nullptr || g == nullptr || ws == nullptr) return kErrNull;
  const Mat mw{w, R, C, ldw, 4}, mg{g, R, C, ldg, in_esize(gt)};
  int st;
  if ((st = check_mat(mw, true)) != kOk) return st;
  if ((st = check_mat(mg, true)) != kOk) return st;
  if (!aligned16(ws) || (norms != nullptr && !aligned4(norms))) return kErrAlign;
  if (ws_bytes < ws_needed) return kErrWorkspace;
  const Mat mws{ws, 1, (int64_t)ws_needed, (int64_t)ws_needed, 1}, mn{norms, 1, 2, 2, 4};
  if (overlaps(mw, mg) || overlaps(mws, mw) || overlaps(mws, mg)) return kErrOverlap;
  if (norms != nullptr && (overlaps(mn, mw) || overlaps(mn, mg) || overlaps(mn, mws))) return kErrOverlap;
  return kOk;
}

int validate_hyperball_batch(const HyperballJobArgs* jobs, int count, int max_jobs, int gt, double lr, double wd,
                             double eps, const void* ws, size_t ws_bytes, size_t ws_needed, bool* empty) {
  if (count < 0 || count > max_jobs) return kErrValue;
  if (count > 0 && jobs == nullptr) return kErrNull;
  if (in_esize(gt) == 0) return kErrDtype;
  if (!finite_nonneg(lr) || !finite_nonneg(wd) || !(finite_nonneg(eps) && eps > 0.0)) return kErrValue;
  bool any = false;
  for (int j = 0; j < count; ++j) {
    const HyperballJobArgs& a = jobs[j];
    // each job alone, with a stand-in workspace (the batch's is checked once below)
    alignas(16) static const double kStandIn[2] = {0.0, 0.0};
    int st = validate_hyperball(a.w, a.ldw, a.g, gt, a.ldg, a.R, a.C, lr, wd, eps, a.radius, a.norms, kStandIn,
                                ws_needed, 0, &empty[j]);
    if (st != kOk) return st;
    any = any || !empty[j];
  }
  if (!any) return kOk;
  if (ws == nullptr) return kErrNull;
  if (!aligned16(ws)) return kErrAlign;
  if (ws_bytes < ws_needed) return kErrWorkspace;
  const Mat mws{ws, 1, (int64_t)ws_needed, (int64_t)ws_needed, 1};
  const int es = in_esize(gt);
  for (int j = 0; j < count; ++j) {
    if (empty[j]) continue;
    const HyperballJobArgs& a = jobs[j];
    const Mat wj{a.w, a.R, a.C, a.ldw, 4}, gj{a.g, a.R, a.C, a.ldg, es}, nj{a.norms, 1, 2, 2, 4};
    if (overlaps(wj, mws) || overlaps(gj, mws) || (a.norms && overlaps(nj, mws))) return kErrOverlap;
    for (int k = 0; k < count; ++k) {
      if (k == j || empty[k]) continue;
      const HyperballJobArgs& b = jobs[k];
      const Mat wk{b.w, b.R, b.C, b.ldw, 4}, gk{b.g, b.R, b.C, b.ldg, es}, nk{b.norms, 1, 2, 2, 4};
      // job j writes w and norms: neither may touch anything job k reads or writes
      if (overlaps(wj, wk) || overlaps(wj, gk) || (b.norms && overlaps(wj, nk))) return kErrOverlap;
      if (a.norms && (overlaps(nj, wk) || overlaps(nj, gk) || (b.norms && overlaps(nj, nk)))) return kErrOverlap;
    }
  }
  return kOk;
}

int validate_stream_copy(const void* src, const void* dst, size_t bytes, bool* empty) {
  *empty = false;
  if (bytes % 16 != 0 || bytes >= ((size_t)1 << 48)) return kErrShape;
  if (bytes == 0) {
    *empty = true;
    return kOk;
  }
  if (!src || !dst) return kErrNull;
  if (!aligned16(src) || !aligned16(dst)) return kErrAlign;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return kErrOverlap;
  return kOk;
}

int validate_gemm(const GemmArgs& g, size_t ws_needed, bool* empty, bool* zero_fill) {
  *empty = false;
  *zero_fill = false;
  if (g.op < 0 || g.op > 4) return kErrShape;
  if (!fmt_ok(g.fa) || !fmt_ok(g.fb)) return kErrFormat;
  if (g.out_t != 0 && g.out_t != 1 && !(g.out_t == 2 && g.op == 2)) return kErrDtype;
  const int64_t M = g.M, N = g.N, K = g.K;
  if (M < 0 || N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return kErrShape;
  if (g.op == 2 && M % 128 != 0) return kErrShape;

  // Operand geometry per op: (A codes, A scales, B codes, B scales, output) as matrices.
  Mat qa, sa, qb, sb, out;
  int64_t out_rows, out_cols, contraction;
  const int oes = g.out_t == 0 ? 2 : 4;
  if (g.op == 4) {  // per-tensor scales: A[M,K], B[N,K] (one scale each) -> Y[M,N]
    qa = Mat{g.qa, M, K, g.ldqa, 1};
    sa = Mat{g.sa, 1, 1, 1, 4};
    qb = Mat{g.qb, N, K, g.ldqb, 1};
    sb = Mat{g.sb, 1, 1, 1, 4};
    out_rows = M; out_cols = N; contraction = K;
  } else if (g.op == 0) {  // fprop: X[M,K] (1x128), W[N,K] (128x128) -> Y[M,N]
    qa = Mat{g.qa, M, K, g.ldqa, 1};
    sa = Mat{g.sa, K / 128, M, g.ldsa, 4};
    qb = Mat{g.qb, N, K, g.ldqb, 1};
    sb = Mat{g.sb, N / 128, K / 128, g.ldsb, 4};
    out_rows = M; out_cols = N; contraction = K;
  } else if (g.op == 3) {  // dgrad on W^T codes: dY[M,N] (1x128), W^T[K,N] (128x128) -> dX[M,K]
    qa = Mat{g.qa, M, N, g.ldqa, 1};
    sa = Mat{g.sa, N / 128, M, g.ldsa, 4};
    qb = Mat{g.qb, K, N, g.ldqb, 1};
    sb = Mat{g.sb, N / 128, K / 128, g.ldsb, 4};
    out_rows = M; out_cols = K; contraction = N;
  } else if (g.op == 1) {  // dgrad: dY[M,N] (1x128), W[N,K] (128x128) -> dX[M,K]
    qa = Mat{g.qa, M, N, g.ldqa, 1};
    sa = Mat{g.sa, N / 128, M, g.ldsa, 4};
    qb = Mat{g.qb, N, K, g.ldqb, 1};
    sb = Mat{g.sb, N / 128, K / 128, g.ldsb, 4};
    out_rows = M; out_cols = K; contraction = N;
  } else {  // wgrad: dY^T[N,M] (128x1), X^T[K,M] (128x1) -> dW[N,K]
    qa = Mat{g.qa, N, M, g.ldqa, 1};
    sa = Mat{g.sa, M / 128, N, g.ldsa, 4};
    qb = Mat{g.qb, K, M, g.ldqb, 1};
    sb = Mat{g.sb, M / 128, K, g.ldsb, 4};
    out_rows = N; out_cols = K; contraction = M;
  }
  out = Mat{g.out, out_rows, out_cols, g.ldout, oes};
  if (out_rows == 0 || out_cols == 0) {
    *empty = true;
    return kOk;
  }
  int st;
  if (g.out == nullptr) return kErrNull;
  if ((st = check_mat(out, true)) != kOk) return st;
  if (contraction == 0) {
    *zero_fill = true;
    return kOk;
  }
  if (g.qa == nullptr || g.sa == nullptr || g.qb == nullptr || g.sb == nullptr) return kErrNull;
  if ((st = check_mat(qa, true)) != kOk) return st;
  if ((st = check_mat(qb, true)) != kOk) return st;
  // The kernels reach one tile of a code operand (at most 256 rows of the contraction) through a
  // buffer range of 32 bits: 255 row strides plus one row must stay below 4 GiB.  (dgrad's W codes
  // are first transposed into the workspace with rows of N bytes.)
  const int64_t kSpan = (int64_t)1 << 32;
  if (255 * qa.ld + contraction >= kSpan) return kErrLd;
  if (g.op != 1 && 255 * qb.ld + contraction >= kSpan) return kErrLd;
  if (g.op == 4) {  // the two scales are single floats
    if (!aligned4(g.sa) || !aligned4(g.sb)) return kErrAlign;
  } else {
    if ((st = check_mat(sa, true)) != kOk) return st;
    // weight scales are read one value at a time; the wgrad column scales as 16-byte vectors
    if ((st = check_mat(sb, g.op == 2)) != kOk) return st;
  }
  if (overlaps(out, qa) || overlaps(out, sa) || overlaps(out, qb) || overlaps(out, sb)) return kErrOverlap;
  if (ws_needed > 0) {
    if (g.ws == nullptr || g.ws_bytes < ws_needed) return kErrWorkspace;
    if (!aligned16(g.ws)) return kErrAlign;
    Mat wsm{g.ws, 1, (int64_t)ws_needed, (int64_t)ws_needed, 1};
    if (overlaps(wsm, out) || overlaps(wsm, qa) || overlaps(wsm, sa) || overlaps(wsm, qb) || overlaps(wsm, sb))
      return kErrOverlap;
  }
  return kOk;
}

}  // namespace fp8bq
