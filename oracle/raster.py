"""Per-tile front-to-back compositing and its backward (oracle).

[PROFILE] names the forward kernel ``rasterize_fwd``; [BWD] section 4
describes the backward ``rasterize_to_pixels_3dgs_bwd``: it reuses what the
forward saved (tile offsets, the flattened intersection list, each pixel's
last contributing Gaussian ``last_ids`` and its transmittance
``render_Ts``), splits every pixel's gradient over the Gaussians on it in
proportion to their alpha contribution along the blend order, and sums
the per-pixel contributions into one screen-space gradient per visible
pair.

Readings for the per-pixel rule (the pages give none), for pixel centre
(px, py) and the entries of its tile in sorted order:
  d = (u - px, v - py); sigma = 1/2 (a dx^2 + c dy^2) + b dx dy;
  skip the entry if sigma < 0; alpha = min(0.99, o exp(-sigma));
  skip if alpha < 1/255; T' = T (1 - alpha); if T' < 1e-4 stop *without*
  compositing this entry; else C += rgb alpha T, T = T', last = index.
Output: premultiplied colour, final T, and ``last`` as the local index
within the tile's range (-1 when nothing was composited).

Depth channel and background ([BWD] section 2: the per-pixel output
gradients are v_render_rgb, v_render_depth and v_render_Ts; section 3:
the background blend's backward hook adds its transmittance gradient into
v_render_Ts). Readings: the rendered depth is composited like a colour
channel whose value is the entry's depth z (D = sum z alpha T, not
normalised); the background is one RGB colour per camera added as
C_out = C + T_final bg, absent (zero) when not given.

Backward, for L = <v_rgb, C_out> + <v_T, T_final> + <v_depth, D> and
composited entry i at a pixel, with T_i the transmittance before i,
S_i = sum_{j>i} c_j a_j T_j and S^D_i = sum_{j>i} z_j a_j T_j:
  dL/drgb_i  = a_i T_i v_rgb,  dL/dz_i = a_i T_i v_depth
  dL/da_i    = v_rgb . (c_i T_i - S_i / (1 - a_i))
               + v_depth (z_i T_i - S^D_i / (1 - a_i))
               - (v_T + v_rgb . bg) T_final / (1 - a_i)
  dL/dbg     = sum over the camera's pixels of v_rgb T_final
  dL/do      = dL/da e^-sigma,  dL/dsigma = -dL/da a  (both 0 when the 0.99
               clamp is active), and sigma's partials in (u, v, a, b, c).
The discrete decisions (skips, the stop, the clamp) are not differentiated.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rasterize_fwd", "rasterize_bwd", "background_grad", "ALPHA_MIN", "ALPHA_MAX",
           "T_STOP"]

TILE = 16
ALPHA_MIN = 1.0 / 255.0
ALPHA_MAX = 0.99
T_STOP = 1e-4


def _tile_pixels(t_local: int, tiles_x: int, W: int, H: int):
    ty, tx = divmod(t_local, tiles_x)
    ys = np.arange(ty * TILE, min(H, ty * TILE + TILE))
    xs = np.arange(tx * TILE, min(W, tx * TILE + TILE))
    ii, jj = np.meshgrid(ys, xs, indexing="ij")
    return ii.ravel(), jj.ravel()


def _walk_tile(rows: np.ndarray, px: np.ndarray, py: np.ndarray, record: bool):
    """Composite one tile's entries over its pixels, entry by entry."""
    P, n = px.size, rows.shape[0]
    T = np.ones(P)
    C = np.zeros((P, 4))   # rgb and depth
    last = np.full(P, -1, np.int64)
    evals = np.zeros(P, np.int64)
    active = np.ones(P, bool)
    rec = None
    if record:
        rec = dict(alpha=np.zeros((P, n)), Tb=np.zeros((P, n)), comp=np.zeros((P, n), bool),
                   ex=np.zeros((P, n)), clamp=np.zeros((P, n), bool),
                   dx=np.zeros((P, n)), dy=np.zeros((P, n)))
    for j in range(n):
        if not active.any():
            break
        u, v, a, b, c, o = rows[j, :6]
        rgbz = rows[j, [7, 8, 9, 6]]
        dx = u - px
        dy = v - py
        sigma = 0.5 * (a * dx * dx + c * dy * dy) + b * dx * dy
        ex = np.exp(-sigma)
        raw_alpha = o * ex
        alpha = np.minimum(ALPHA_MAX, raw_alpha)
        evals += active
        ok = active & (sigma >= 0.0) & (alpha >= ALPHA_MIN)
        Tn = T * (1.0 - alpha)
        stop = ok & (Tn < T_STOP)
        active &= ~stop
        ok &= ~stop
        if record:
            rec["alpha"][:, j] = alpha
            rec["Tb"][:, j] = T
            rec["comp"][:, j] = ok
            rec["ex"][:, j] = ex
            rec["clamp"][:, j] = raw_alpha > ALPHA_MAX
            rec["dx"][:, j] = dx
            rec["dy"][:, j] = dy
        C[ok] += rgbz[None, :] * (alpha[ok] * T[ok])[:, None]
        T = np.where(ok, Tn, T)
        last[ok] = j
    return C, T, last, evals, rec


def _tile_list(tile_offsets, flatten_ids, t):
    return np.asarray(flatten_ids[int(tile_offsets[t]):int(tile_offsets[t + 1])], np.int64)


def rasterize_fwd(screen, flatten_ids, tile_offsets, C: int, W: int, H: int, tiles=None,
                  background=None, depth: bool = False):
    """(out_rgb[C,H,W,3], out_T[C,H,W], last_ids[C,H,W], evals[C,H,W]),
    plus out_depth[C,H,W] last when ``depth`` is set.

    ``tiles``: optional iterable of global tile ids (c * T + local) to
    evaluate; other pixels are left NaN (last_ids -2, evals -1).
    ``background``: optional [C, 3] colour blended in as C + T_final bg.
    """
    tiles_x, tiles_y = (W + TILE - 1) // TILE, (H + TILE - 1) // TILE
    T_per = tiles_x * tiles_y
    out_rgb = np.full((C, H, W, 3), np.nan)
    out_T = np.full((C, H, W), np.nan)
    out_depth = np.full((C, H, W), np.nan)
    last_ids = np.full((C, H, W), -2, np.int64)
    evals = np.full((C, H, W), -1, np.int64)
    screen = np.asarray(screen, np.float64)
    bg = None if background is None else np.asarray(background, np.float64).reshape(C, 3)
    for t in (range(C * T_per) if tiles is None else tiles):
        c, tl = divmod(int(t), T_per)
        ii, jj = _tile_pixels(tl, tiles_x, W, H)
        ids = _tile_list(tile_offsets, flatten_ids, t)
        Cc, Tt, last, ev, _ = _walk_tile(screen[ids], jj + 0.5, ii + 0.5, record=False)
        rgb = Cc[:, :3] if bg is None else Cc[:, :3] + Tt[:, None] * bg[c][None, :]
        out_rgb[c, ii, jj] = rgb
        out_depth[c, ii, jj] = Cc[:, 3]
        out_T[c, ii, jj] = Tt
        last_ids[c, ii, jj] = last
        evals[c, ii, jj] = ev
    if depth:
        return out_rgb, out_T, last_ids, evals, out_depth
    return out_rgb, out_T, last_ids, evals


def rasterize_bwd(screen, flatten_ids, tile_offsets, C: int, W: int, H: int,
                  v_rgb, v_T=None, tiles=None, v_depth=None, background=None):
    """dL/d(screen rows) [nnz, 10] for L = <v_rgb, out_rgb> + <v_T, out_T>
    + <v_depth, out_depth>.

    The depth column of the result is 0 when ``v_depth`` is None (the
    colour image does not depend on it). ``background`` is the forward's
    [C, 3] colour (None = no blend). ``tiles`` restricts the sum to those
    global tile ids.
    """
    tiles_x, tiles_y = (W + TILE - 1) // TILE, (H + TILE - 1) // TILE
    T_per = tiles_x * tiles_y
    screen = np.asarray(screen, np.float64)
    v_screen = np.zeros_like(screen)
    v_rgb = np.asarray(v_rgb, np.float64)
    v_T = np.zeros(v_rgb.shape[:3]) if v_T is None else np.asarray(v_T, np.float64)
    v_D = np.zeros(v_rgb.shape[:3]) if v_depth is None else np.asarray(v_depth, np.float64)
    if background is not None:
        # the background hook: T_final also feeds C_out through T bg
        bg = np.asarray(background, np.float64).reshape(C, 3)
        v_T = v_T + np.einsum("chwk,ck->chw", v_rgb, bg)
    for t in (range(C * T_per) if tiles is None else tiles):
        c, tl = divmod(int(t), T_per)
        ii, jj = _tile_pixels(tl, tiles_x, W, H)
        ids = _tile_list(tile_offsets, flatten_ids, t)
        if ids.size == 0:
            continue
        rows = screen[ids]
        px, py = jj + 0.5, ii + 0.5
        _, Tfin, last, _, rec = _walk_tile(rows, px, py, record=True)
        n_used = int(last.max()) + 1
        if n_used <= 0:
            continue
        rows = rows[:n_used]
        ids = ids[:n_used]
        comp = rec["comp"][:, :n_used]
        alpha = rec["alpha"][:, :n_used]
        Tb = rec["Tb"][:, :n_used]
        ex = rec["ex"][:, :n_used]
        clamp = rec["clamp"][:, :n_used]
        dx, dy = rec["dx"][:, :n_used], rec["dy"][:, :n_used]
        # the depth is a fourth channel with value z and upstream v_depth
        gr = np.concatenate([v_rgb[c, ii, jj], v_D[c, ii, jj][:, None]], 1)   # [P, 4]
        gT = v_T[c, ii, jj]              # [P]
        chan = rows[:, [7, 8, 9, 6]]                       # [n, 4]
        w = np.where(comp, alpha * Tb, 0.0)               # [P, n]
        contrib = w[:, :, None] * chan[None]               # [P, n, 4]
        suffix = np.cumsum(contrib[:, ::-1], axis=1)[:, ::-1]
        S = suffix - contrib                               # sum over j > i
        one_m = 1.0 - alpha
        v_alpha = (np.einsum("pc,pnc->pn", gr, chan[None] * Tb[:, :, None] - S / one_m[:, :, None])
                   - gT[:, None] * Tfin[:, None] / one_m)
        v_alpha = np.where(comp, v_alpha, 0.0)
        free = comp & ~clamp
        v_sigma = np.where(free, -v_alpha * alpha, 0.0)
        v_o = np.where(free, v_alpha * ex, 0.0)
        a, b, cc = rows[:, 2], rows[:, 3], rows[:, 4]
        g = np.zeros((n_used, 10))
        g[:, 0] = (v_sigma * (a[None] * dx + b[None] * dy)).sum(0)
        g[:, 1] = (v_sigma * (b[None] * dx + cc[None] * dy)).sum(0)
        g[:, 2] = (v_sigma * 0.5 * dx * dx).sum(0)
        g[:, 3] = (v_sigma * dx * dy).sum(0)
        g[:, 4] = (v_sigma * 0.5 * dy * dy).sum(0)
        g[:, 5] = v_o.sum(0)
        g[:, 7:10] = np.einsum("pn,pc->nc", w, gr[:, :3])
        g[:, 6] = np.einsum("pn,p->n", w, gr[:, 3])
        np.add.at(v_screen, ids, g)
    return v_screen


def background_grad(out_T, v_rgb):
    """dL/dbg [C, 3] of the blend C + T_final bg: sum over each camera's
    pixels of v_rgb T_final."""
    return np.einsum("chwk,chw->ck", np.asarray(v_rgb, np.float64), np.asarray(out_T, np.float64))


def decision_signature(screen, flatten_ids, tile_offsets, C: int, W: int, H: int) -> bytes:
    """Every discrete decision of the forward, for finite-difference guards:
    per tile and pixel, which entries were composited and which hit the 0.99
    clamp (the stop decision is implied by the composited set)."""
    import hashlib
    tiles_x, tiles_y = (W + TILE - 1) // TILE, (H + TILE - 1) // TILE
    h = hashlib.sha1()
    h.update(np.asarray(flatten_ids, np.int64).tobytes())
    h.update(np.asarray(tile_offsets, np.int64).tobytes())
    screen = np.asarray(screen, np.float64)
    for t in range(C * tiles_x * tiles_y):
        _, tl = divmod(t, tiles_x * tiles_y)
        ii, jj = _tile_pixels(tl, tiles_x, W, H)
        ids = _tile_list(tile_offsets, flatten_ids, t)
        if ids.size == 0:
            continue
        _, _, _, _, rec = _walk_tile(screen[ids], jj + 0.5, ii + 0.5, record=True)
        h.update(np.packbits(rec["comp"]).tobytes())
        h.update(np.packbits(rec["comp"] & rec["clamp"]).tobytes())
    return h.digest()
