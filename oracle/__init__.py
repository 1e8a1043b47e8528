"""Plain fp64 CPU oracle for the OCTOPUS key codec.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and shares no code, table or constant generator with it.

Everything here is written from the method description on the pages:

* [YL]  youleyou.com Chinese summary of arXiv:2605.21226 (OCTOPUS), cited by
        its section headings (旋转魔法, 八面体折叠, 三元组分解, 非均匀比特分配,
        联合取整, 实验结果, 可选的残差修正, 工程实现).
* [AR]  agents-report.net "OCTOPUS：八面體參數化與 triplet 聯合量化優化
        Transformer KV 快取", cited by section (方法概覽, 位元分配, 實作要點,
        OCTOPUS-QJL).
* [AB]  the paper's abstract (arxivlens / chatpaper pages).
* [TQ]  zhichai.net blog on TurboQuant (prior codec), section 四/五 on QJL.
"""
from .octopus import *  # noqa: F401,F403
