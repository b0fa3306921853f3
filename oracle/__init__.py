"""CPU oracle for the Geometric Context Attention (GCA) step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the package smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants) and it never
imports that library.

Everything is plain numpy in float64.  Inputs arrive as exact upcasts of the
fp32 / bf16 tensors fed to the GPU.

Sources (pages about LingBot-Map, cited by title and section):
  * gitcode.csdn.net technical summary of lingbot-map ("the technical
    summary"): §2.2 frame-type table, §2.3 summary-token table, §2.4 Total
    Tokens equation and its worked comparison table, §2.5 attention-mask
    table and complexity table.
  * "LingBot-Map 论文精读 ..." (lshu.cn, "the paper-to-code map"): §二 2.1
    anchor context, 2.3 trajectory memory (compressing eviction), 2.4 token
    budget; §五 inference system.
  * "LingBot-Map 深度解析 ..." (e.mffb.com.cn, "the deep dive"): §3.2
    streaming main loop, §3.4 paged KV cache.
  * "萬幀實時！流式3D重建天花板..." (m.serenwang.com, "the news article"):
    the attention-mask comparison figure caption (full / causal / sliding /
    GCA with n=2, k=2).

Parity status per function is stated in each module header.
"""
