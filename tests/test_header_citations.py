"""Every compute entry point declared in include/dmoe.h carries a "Source:" line
in its comment that names the page passage defining the operation, or says
that the pages are silent and states the reading taken (no GPU)."""
import os
import re

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dmoe.h")

PAGES = ('Transformers documentation "Dots 3 Note Preview"', "Transformers PR #47844",
         'model card "dots-studio/dots3-note-prev"', 'SGLang cookbook "Dots3-Note"', "orcarouter")


def _entry_points():
    text = open(HEADER).read()
    for m in re.finditer(r"^dmoe_status (dmoe_\w+)\(", text, re.M):
        start = text.rfind("/*", 0, m.start())
        end = text.find("*/", start)
        assert 0 <= start < end < m.start(), f"{m.group(1)} has no comment block before it"
        yield m.group(1), text[start:end]


def test_every_entry_point_cites_its_passage():
    names = []
    for name, comment in _entry_points():
        names.append(name)
        if name == "dmoe_forward_noalloc":  # not a step of the layer: its comment names the callers it serves
            assert "cannot allocate" in " ".join(line.strip(" *") for line in comment.splitlines())
            continue
        src = comment[comment.find("Source:"):] if "Source:" in comment else ""
        assert src, f"{name}: no Source: line"
        src = " ".join(line.strip(" *") for line in src.splitlines())
        ok = any(p in src for p in PAGES) or "pages do not" in src or re.match(r"Source: as dmoe_\w+", src)
        assert ok, f"{name}: Source: line names no page passage: {src[:120]}"
    # the calls of the layer's statement are all there
    for call in ("dmoe_router_logits", "dmoe_route", "dmoe_permute", "dmoe_quant_act", "dmoe_grouped_gemm_gateup",
                 "dmoe_grouped_gemm_down", "dmoe_shared_expert", "dmoe_combine", "dmoe_forward"):
        assert call in names, call


def test_docs_page_cited_by_its_title():
    text = open(HEADER).read()
    assert 'docs "Dots3Note"' not in text and '"Dots3Note"' not in text
