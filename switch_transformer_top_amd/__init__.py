"""Switch FFN layer forward pass for MI355X (gfx950): HIP kernels behind a C ABI.

    from switch_transformer_top_amd import binding
    layer = binding.SwitchLayer(cfg, W_r, b_r, W_in, W_out)

The compiled library is ``lib/libswitch_layer.so`` (built by ``build.py``);
``binding`` refuses to import without it.  The binding is imported on first
use so that ``build`` can run before anything is compiled.
"""


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
